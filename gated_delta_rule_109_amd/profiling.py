"""HBM traffic of the prefill from rocprofv3 byte counters.

rocprofv3 reports FETCH_SIZE and WRITE_SIZE (KiB per dispatch) from the L2
channels. Their scale is calibrated against a plain elementwise kernel of
known size run in the same process: ``bench.py --calibrate MIB`` runs
``torch.abs`` (an op nothing else in the run uses) over a float32 tensor of
MIB MiB, which reads and writes exactly MIB MiB, so each counter is scaled by
the true size over what it reads for that kernel.

It also renders the per-kernel time table of a ``rocprofv3 --kernel-trace
--stats`` run (``--stats DIR``), and the MFMA utilisation of a counter pass
with SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_BF16 and
GRBM_GUI_ACTIVE (``--mfma DIR``), and the memory-pipe counters of two passes
(``--pipe DIR_A DIR_B``: L1-to-L2 read requests and their latency, L1 stalls
on pending L2 data, TA address stalls, L2 hits and misses).

Usage (two counter passes of the same command, then the summary):

  rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dirF> -o kda -- python3 bench.py ... --calibrate 256
  rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dirW> -o kda -- python3 bench.py ... --calibrate 256
  python3 -m gated_delta_rule_109_amd.profiling --fetch <dirF> --write <dirW> --calib-mib 256 \
      --out profiles/<name>.md --command "<the rocprofv3 command>"

The summary ends with one ``traffic-record:`` JSON line that bench.py reads:
the per-call HBM bytes of kda_prefill_chunked and a digest of the kernel
sources it was measured on (a changed source makes bench.py report null).
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
CHIP_CUS = 256                                # MI355X compute units


RECORD_BYTES = 47 * 1024                      # one block record at D = 128
SINGLE_SEQ_WINDOW_BYTES = 1 << 30             # records per window of a one-sequence call


def prefill_windows(num_seqs, heads, blocks):
    """Blocks per record window of a call whose workspace holds all of its
    records (kda_prefill_workspace_size's): one window, except that a single
    sequence takes windows of about 1 GiB of records, evened out."""
    if num_seqs != 1:
        return [blocks]
    w = max(1, min(SINGLE_SEQ_WINDOW_BYTES // (heads * RECORD_BYTES), 65535))
    if blocks <= w:
        return [blocks]
    nwin = -(-blocks // w)
    w = -(-blocks // nwin)
    return [w] * (nwin - 1) + [blocks - w * (nwin - 1)]


def prefill_kernels(heads, blocks, units, num_seqs=None):
    """The kernels of one plain kda_prefill_chunked call at D = 128 (bf16 q/k/v,
    no front end, no segments) with `blocks` 32-token blocks per head and
    `units` (sequence, head) chain units, as ((kernel, grid in work-items),
    dispatches per call) (the same instantiations also run other shapes in
    the same program, so a dispatch is selected by kernel and grid). Every
    record window runs one prep and one chain dispatch; windows of a single
    sequence hold all of its units."""
    num_seqs = units // heads if num_seqs is None else num_seqs
    groups = (units + 7) // 8                 # 8 units x (slice groups) per group of workgroups
    if units * 8 > CHIP_CUS:                  # more 16-column slices than CUs: two per workgroup
        chain = ("kda::chain_kernel<128, unsigned short, 2, false>", groups * 8 * 4 * 512)
    else:
        chain = ("kda::chain_kernel<128, unsigned short, 1, false>", groups * 8 * 8 * 448)
    windows = prefill_windows(num_seqs, heads, blocks)
    out = {("kda::plan_kernel", 1024): 1}
    for w in windows:
        key = ("kda::prep_kernel<128, unsigned short, false, false>", heads * w * 128)
        out[key] = out.get(key, 0) + 1
    out[chain] = len(windows)
    return tuple(out.items())


# B = 1, H = 32, T = 131072 (4096 blocks) and T = 8192 (256 blocks); 16 packed
# sequences of 87,687 tokens (2748 blocks), H = 32
PREFILL_LONG = prefill_kernels(32, 4096, 32)
PREFILL_8K = prefill_kernels(32, 256, 32)
PREFILL_VARLEN = prefill_kernels(32, 2748, 16 * 32, num_seqs=16)
PREFILL_KERNELS = PREFILL_LONG
# one kda_decode_step over 256 sequences x 32 heads at D = 128 (one workgroup of
# 256 threads per head)
DECODE_KERNELS = ((("kda::decode_kernel<128, unsigned short, true, false>", 256 * 32 * 256), 1),)
WORKLOADS = {
    "prefill": (PREFILL_LONG, "KDA prefill HBM traffic (B=1, H=32, T=131072, D=128, checkpoint every 32768, "
                "bf16 q/k/v)", "kda_prefill_chunked"),
    "prefill_8k": (PREFILL_8K, "KDA prefill HBM traffic (B=1, H=32, T=8192, D=128, bf16 q/k/v)",
                   "kda_prefill_chunked"),
    "varlen": (PREFILL_VARLEN, "KDA prefill HBM traffic (16 packed sequences, 87687 tokens, H=32, D=128, "
               "cached initial states, bf16 q/k/v)", "kda_prefill_chunked"),
    "decode": (DECODE_KERNELS, "KDA decode HBM traffic (256 sequences x 32 heads, D=128, one token, bf16 q/k/v)",
               "kda_decode_step"),
}
CALIB_KERNEL = "AbsFunctor"


def _code_only(text):
    """Source text without comments and with whitespace collapsed: a comment
    or layout change leaves the compiled kernels, and so the digest, alone."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest():
    """sha256 over the code (comments dropped) of the HIP sources and headers
    the library is built from, and of the public header."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")) + glob.glob(os.path.join(PKG, "csrc", "*.h")))
    files.append(os.path.join(os.path.dirname(PKG), "include", "kda.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def _counter_csv(d):
    hits = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not hits:
        raise FileNotFoundError(f"no counter_collection.csv under {d}")
    return hits[0]


def kernel_key(name):
    """A kernel's name with its template arguments, without the parameter list."""
    return re.sub(r"\(.*", "", name).replace("void ", "").strip()


def per_kernel(d, counter):
    """{(kernel name with template arguments, grid work-items): (dispatches,
    mean KiB per dispatch)} for one counter."""
    acc = {}
    for r in csv.DictReader(open(_counter_csv(d))):
        if r["Counter_Name"] != counter:
            continue
        name = r["Kernel_Name"]
        grid = int(float(r.get("Grid_Size") or 0))
        if "kda::" in name:
            key = (kernel_key(name), grid)
        elif CALIB_KERNEL in name:
            key = (CALIB_KERNEL, 0)
        else:
            continue
        n, s = acc.get(key, (0, 0.0))
        acc[key] = (n + 1, s + float(r["Counter_Value"]))
    return {k: (n, s / n) for k, (n, s) in acc.items()}


def summarize(fetch_dir, write_dir, calib_mib, kernels=PREFILL_KERNELS):
    f = per_kernel(fetch_dir, "FETCH_SIZE")
    w = per_kernel(write_dir, "WRITE_SIZE")
    calib_kib = calib_mib * 1024.0
    cal = (CALIB_KERNEL, 0)
    if cal not in f or cal not in w:
        raise RuntimeError("calibration kernel missing from the counter runs (run bench.py with --calibrate)")
    ff = calib_kib / f[cal][1]     # true bytes per counted byte
    fw = calib_kib / w[cal][1]
    rows = []
    total = 0.0
    mine = dict(kernels)
    for k, per_call in kernels:
        if k not in f or k not in w:
            raise RuntimeError(f"{k} missing from the counter runs")
        fb = f[k][1] * ff * 1024
        wb = w[k][1] * fw * 1024
        total += (fb + wb) * per_call
        rows.append((k, f[k][0], f[k][1], w[k][1], fb, wb, per_call))
    others = [(k, f[k][0], f[k][1], w[k][1], f[k][1] * ff * 1024, w[k][1] * fw * 1024)
              for k in sorted(f) if k in w and k not in mine and k != cal]
    return {"fetch_factor": ff, "write_factor": fw, "rows": rows, "others": others,
            "bytes_per_call": total, "calib": (f[cal][1], w[cal][1])}


def render(res, calib_mib, command, algorithmic_bytes, title=WORKLOADS["prefill"][1],
           call=WORKLOADS["prefill"][2]):
    out = [f"# {title}", "",
           "Commands (run from the repository root on one MI355X; one counter per pass):", "", "```"]
    out += [c for c in command]
    out += ["```", "",
            f"Calibration: `torch.abs` over a {calib_mib} MiB float32 tensor reads and writes exactly "
            f"{calib_mib} MiB; the counters read {res['calib'][0]:.4g} KiB (FETCH_SIZE) and "
            f"{res['calib'][1]:.4g} KiB (WRITE_SIZE), so FETCH_SIZE is scaled by {res['fetch_factor']:.3f} "
            f"and WRITE_SIZE by {res['write_factor']:.3f}.", "",
            "Per dispatch of each kernel and grid (a call runs one prep and one chain dispatch per record "
            "window):", "",
            "| kernel | grid (work-items) | dispatches | per call | FETCH_SIZE KiB | WRITE_SIZE KiB | read MB (scaled) | written MB (scaled) |",
            "|---|---|---|---|---|---|---|---|"]
    for (k, grid), n, fk, wk, fb, wb, per_call in res["rows"]:
        out.append(f"| `{k}` | {grid} | {n} | {per_call} | {fk:.4g} | {wk:.4g} | {fb / 1e6:.1f} | {wb / 1e6:.1f} |")
    tot = res["bytes_per_call"]
    if res.get("others"):
        out += ["", "Other kda kernels in the same run (not part of the call above; per dispatch):", "",
                "| kernel | grid (work-items) | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read MB (scaled) | written MB (scaled) |",
                "|---|---|---|---|---|---|---|"]
        for (k, grid), n, fk, wk, fb, wb in res["others"]:
            out.append(f"| `{k}` | {grid} | {n} | {fk:.4g} | {wk:.4g} | {fb / 1e6:.1f} | {wb / 1e6:.1f} |")
    out += ["", f"HBM bytes per `{call}` call: {tot / 1e6:.1f} MB, against "
            f"{algorithmic_bytes / 1e6:.1f} MB algorithmic (ratio {tot / algorithmic_bytes:.2f}).", "",
            "traffic-record: " + json.dumps({"bytes_per_call": round(tot), "source_digest": source_digest(),
                                              "fetch_factor": round(res["fetch_factor"], 4),
                                              "write_factor": round(res["write_factor"], 4)})]
    return "\n".join(out) + "\n"


def read_record(path):
    """The traffic-record of a summary if it matches the current sources, else None."""
    try:
        for line in open(path):
            if line.startswith("traffic-record: "):
                rec = json.loads(line[len("traffic-record: "):])
                return rec if rec.get("source_digest") == source_digest() else None
    except OSError:
        return None
    return None


def kernel_stats(d):
    """[(name, grid work-items, calls, avg us, min us, max us, share %)] of the
    kda kernels, one row per kernel and grid, from the per-dispatch
    kernel_trace.csv of a rocprofv3 --kernel-trace run (share: of all kernel
    time in the trace)."""
    hits = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not hits:
        raise FileNotFoundError(f"no kernel_trace.csv under {d}")
    acc, total = {}, 0.0
    for r in csv.DictReader(open(hits[0])):
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        total += dur
        if "kda::" not in r["Kernel_Name"]:
            continue
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        acc.setdefault((kernel_key(r["Kernel_Name"]), grid), []).append(dur)
    rows = [(k, g, len(v), float(np.mean(v)), min(v), max(v), 100.0 * sum(v) / total)
            for (k, g), v in acc.items()]
    return sorted(rows, key=lambda r: -r[6])


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "GRBM_GUI_ACTIVE")
SIMD_NUM = 256 * 4          # MI355X: 256 CUs x 4 SIMDs
XCD_NUM = 8                 # GRBM_GUI_ACTIVE comes summed over the 8 XCDs
PEAK_KERNEL = "mfma_loop"   # the reference loop of libkda_peak.so


def mfma_summary(d):
    """[(kernel, grid work-items, dispatches, MFMA busy %, bf16 MFMA GFLOP per
    dispatch)], one row per kernel and grid: busy
    cycles over all SIMDs / (GPU-active cycles of one XCD x SIMD_NUM); FLOPs =
    MOPS x 512. The CSV holds GRBM_GUI_ACTIVE summed over the XCDs, so it is
    divided by XCD_NUM (the vendor's MfmaUtil takes its maximum over them)."""
    acc = {}
    for r in csv.DictReader(open(_counter_csv(d))):
        name = r["Kernel_Name"]
        grid = int(float(r.get("Grid_Size") or 0))
        if "kda::" in name:
            key = (kernel_key(name), grid)
        elif PEAK_KERNEL in name:
            key = (kernel_key(name.replace("(anonymous namespace)::", "")) + " (reference loop)", grid)
        else:
            continue
        c = r["Counter_Name"]
        if c not in MFMA_COUNTERS:
            continue
        per = acc.setdefault(key, {}).setdefault(c, [])
        per.append(float(r["Counter_Value"]))
    rows = []
    for key, per in sorted(acc.items()):
        if not all(c in per for c in MFMA_COUNTERS):
            continue
        n = len(per["GRBM_GUI_ACTIVE"])
        busy = np.mean(per["SQ_VALU_MFMA_BUSY_CYCLES"])
        active = np.mean(per["GRBM_GUI_ACTIVE"]) / XCD_NUM
        flops = np.mean(per["SQ_INSTS_VALU_MFMA_MOPS_BF16"]) * 512
        rows.append((key[0], key[1], n, 100.0 * busy / (active * SIMD_NUM), flops / 1e9))
    return rows


PIPE_COUNTERS = ("TCP_TCC_READ_REQ_LATENCY_sum", "TCP_TCC_READ_REQ_sum", "TCP_PENDING_STALL_CYCLES_sum",
                 "TA_ADDR_STALLED_BY_TC_CYCLES_sum", "TCC_HIT_sum", "TCC_MISS_sum", "GRBM_GUI_ACTIVE")
CU_NUM = 256                # MI355X compute units


def pipe_summary(dirs):
    """[(kernel, dispatches, GPU cycles, L2 read requests per CU, mean L2 read
    latency in cycles, share of cycles the L1 stalls on pending L2 data,
    share of cycles the TA address path stalls on the L1, L2 hit rate)] of
    the kda kernels, one row per kernel, from counter passes that together
    hold PIPE_COUNTERS (each pass with its own GRBM_GUI_ACTIVE). Per
    dispatch; GRBM_GUI_ACTIVE is summed over the XCDs in the CSV (divided by
    XCD_NUM here) and the TCP/TA counters over the compute units (divided by
    CU_NUM for the per-CU shares)."""
    vals = {}
    for d in dirs:
        per_disp = {}
        for r in csv.DictReader(open(_counter_csv(d))):
            if "kda::" not in r["Kernel_Name"]:
                continue
            key = (kernel_key(r["Kernel_Name"]), r["Dispatch_Id"])
            per_disp.setdefault(key, {}).setdefault(r["Counter_Name"], 0.0)
            per_disp[key][r["Counter_Name"]] += float(r["Counter_Value"])
        for (k, _), cs in per_disp.items():
            cyc = cs.get("GRBM_GUI_ACTIVE", 0.0) / XCD_NUM
            for c, v in cs.items():
                if c == "GRBM_GUI_ACTIVE":
                    continue
                vals.setdefault(k, {}).setdefault(c, []).append((v, cyc))
            vals.setdefault(k, {}).setdefault("GRBM_GUI_ACTIVE", []).append((cyc, cyc))
    rows = []
    for k, cs in sorted(vals.items()):
        if not all(c in cs for c in PIPE_COUNTERS):
            continue
        mean = lambda c: float(np.mean([v for v, _ in cs[c]]))
        share = lambda c: float(np.mean([v / CU_NUM / cyc for v, cyc in cs[c] if cyc > 0]))
        req = mean("TCP_TCC_READ_REQ_sum")
        if req < CU_NUM:            # kernels with next to no memory traffic (the plan kernel)
            continue
        hits, misses = mean("TCC_HIT_sum"), mean("TCC_MISS_sum")
        rows.append((k, len(cs["TCP_TCC_READ_REQ_sum"]), mean("GRBM_GUI_ACTIVE"), req / CU_NUM,
                     mean("TCP_TCC_READ_REQ_LATENCY_sum") / req, 100.0 * share("TCP_PENDING_STALL_CYCLES_sum"),
                     100.0 * share("TA_ADDR_STALLED_BY_TC_CYCLES_sum"), 100.0 * hits / max(hits + misses, 1.0)))
    return rows


def render_pipe(rows, title, command):
    out = [f"# {title}", "", "Commands (run from the repository root on one MI355X; one pass per counter group):",
           "", "```"]
    out += list(command)
    out += ["```", "",
            "Per dispatch, averaged over the dispatches of each kernel. GRBM_GUI_ACTIVE arrives summed over the "
            "8 XCDs and is divided by 8; the TCP and TA counters are summed over the 256 compute units and are "
            "divided by 256 for the per-CU columns.", "",
            "| kernel | dispatches | GPU cycles | L2 read requests per CU | mean L2 read latency (cycles) | "
            "L1 stalled on pending L2 data (share of cycles, per CU) | TA address path stalled by L1 (share) | "
            "L2 hit rate |", "|---|---|---|---|---|---|---|---|"]
    for k, n, cyc, req, lat, pend, tas, hit in rows:
        out.append(f"| `{k}` | {n} | {cyc:.3g} | {req:.4g} | {lat:.0f} | {pend:.0f} % | {tas:.0f} % | {hit:.0f} % |")
    return "\n".join(out) + "\n"


def render_mfma(rows, title, command):
    out = [f"# {title}", "", "Command (run from the repository root on one MI355X):", "", "```"]
    out += list(command)
    out += ["```", "",
            "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES summed over the SIMDs / (GRBM_GUI_ACTIVE of one XCD x "
            "1024 SIMDs) (the CSV sums GRBM_GUI_ACTIVE over the 8 XCDs); "
            "bf16 MFMA FLOPs = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512. This counts every MFMA the kernels issue "
            "(hi/lo split terms and padding included), not the model FLOPs. The reference loop "
            "(independent MFMA chains, libkda_peak.so; <0> = 16x16x32, <1> = 32x32x16) shows what the counter reads for a matrix-bound kernel.",
            "", "| kernel | grid (work-items) | dispatches | MFMA busy % | bf16 MFMA GFLOP per dispatch |",
            "|---|---|---|---|---|"]
    for key, grid, n, util, gf in rows:
        out.append(f"| `{key}` | {grid} | {n} | {util:.2f} | {gf:.2f} |")
    return "\n".join(out) + "\n"


def render_stats(rows, title, command, bench_line):
    out = [f"# {title}", "", "Command (run from the repository root on one MI355X):", "", "```"]
    out += list(command)
    out += ["```", "", "rocprofv3 kernel statistics of the kda kernels (durations in microseconds; share is "
            "of all GPU kernel time in the run, input generation included):", "",
            "| kernel | grid (work-items) | calls | average | min | max | share |", "|---|---|---|---|---|---|---|"]
    for name, grid, n, avg, mn, mx, pct in rows:
        out.append(f"| `{name}` | {grid} | {n} | {avg:.2f} | {mn:.2f} | {mx:.2f} | {pct:.1f} % |")
    if bench_line:
        out += ["", "bench.py line of the same build (no profiler):", "", "```", bench_line.strip(), "```"]
    return "\n".join(out) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--calib-mib", type=int)
    ap.add_argument("--algorithmic-bytes", type=int)
    ap.add_argument("--stats", help="rocprofv3 --kernel-trace --stats output directory (kernel-time summary)")
    ap.add_argument("--mfma", help="rocprofv3 --pmc output directory with the MFMA counters")
    ap.add_argument("--pipe", nargs="+", help="rocprofv3 --pmc output directories with the memory-pipe counters")
    ap.add_argument("--note", action="append", default=[], help="paragraph appended to the summary")
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="prefill",
                    help="which call the byte-counter summary adds up")
    ap.add_argument("--title", default="KDA kernels")
    ap.add_argument("--bench-line", help="file whose last line is the bench.py JSON line")
    ap.add_argument("--command", action="append", default=[])
    ap.add_argument("--out")
    a = ap.parse_args(argv)
    if a.stats:
        line = open(a.bench_line).read().strip().splitlines()[-1] if a.bench_line else None
        text = render_stats(kernel_stats(a.stats), a.title, a.command, line)
    elif a.mfma:
        text = render_mfma(mfma_summary(a.mfma), a.title, a.command)
    elif a.pipe:
        text = render_pipe(pipe_summary(a.pipe), a.title, a.command)
    else:
        if not (a.fetch and a.write and a.calib_mib and a.algorithmic_bytes):
            ap.error("--fetch, --write, --calib-mib and --algorithmic-bytes are required")
        kernels, title, call = WORKLOADS[a.workload]
        text = render(summarize(a.fetch, a.write, a.calib_mib, kernels), a.calib_mib, a.command,
                      a.algorithmic_bytes, title, call)
    for note in a.note:
        text += "\n" + note.strip() + "\n"
    if a.out:
        with open(a.out, "w") as fh:
            fh.write(text)
    sys.stdout.write(text)


if __name__ == "__main__":
    main()
