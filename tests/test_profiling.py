"""The rocprofv3 summaries behind roofline.traffic and the MFMA figures,
checked on small synthetic counter files (CPU only)."""
import csv
import json
import os

import pytest

from gated_delta_rule_109_amd import profiling as P

FIELDS = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
GRID = {"plan": 1024, "prep": 32 * 4096 * 128, "chain": 256 * 448}   # the long prefill's call


def grid_of(name):
    for key, g in GRID.items():
        if key + "_kernel" in name:
            return g
    return 0


def write_counters(d, rows):
    """rows: (kernel, counter, value[, grid]); the grid defaults to the
    benchmarked call's grid for that kernel."""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "kda_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, FIELDS)
        w.writeheader()
        for i, row in enumerate(rows):
            k, c, v = row[:3]
            grid = row[3] if len(row) > 3 else grid_of(k)
            w.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Grid_Size": grid, "Counter_Name": c,
                        "Counter_Value": v})


PLAN = "kda::plan_kernel(int const*, int)"
PREP = "void kda::prep_kernel<128, unsigned short, false, false>(unsigned short const*)"
PREP_GEN = "void kda::prep_kernel<128, unsigned short, true, false>(unsigned short const*)"
CHAIN = "void kda::chain_kernel<128, unsigned short, 1, false>(unsigned short const*)"
ABS = "void at::native::vectorized_elementwise_kernel<4, at::native::AbsFunctor<float>>(int)"


def test_traffic_summary_scales_by_the_calibration_kernel(tmp_path):
    f, w = str(tmp_path / "f"), str(tmp_path / "w")
    # a call of two record windows: plan once, prep on two grids, chain twice
    P1, P2, C = 32 * 683 * 128, 32 * 681 * 128, 256 * 448
    kernels = ((("kda::plan_kernel", 1024), 1), (("kda::prep_kernel<128, unsigned short, false, false>", P1), 1),
               (("kda::prep_kernel<128, unsigned short, false, false>", P2), 1),
               (("kda::chain_kernel<128, unsigned short, 1, false>", C), 2))
    # the calibration kernel reads and writes 256 MiB; the counters read half
    # of that for FETCH_SIZE and all of it for WRITE_SIZE
    write_counters(f, [(ABS, "FETCH_SIZE", 128 * 1024), (PLAN, "FETCH_SIZE", 1, 1024), (PREP, "FETCH_SIZE", 1000, P1),
                       (PREP, "FETCH_SIZE", 900, P2), (PREP_GEN, "FETCH_SIZE", 5000, P1),
                       (CHAIN, "FETCH_SIZE", 2000, C), (CHAIN, "FETCH_SIZE", 4000, C),
                       (CHAIN, "FETCH_SIZE", 99999, 4 * 8 * 448)])      # a smaller call: not counted
    write_counters(w, [(ABS, "WRITE_SIZE", 256 * 1024), (PLAN, "WRITE_SIZE", 1, 1024), (PREP, "WRITE_SIZE", 300, P1),
                       (PREP, "WRITE_SIZE", 200, P2), (PREP_GEN, "WRITE_SIZE", 9, P1), (CHAIN, "WRITE_SIZE", 100, C)])
    res = P.summarize(f, w, 256, kernels)
    assert res["fetch_factor"] == pytest.approx(2.0) and res["write_factor"] == pytest.approx(1.0)
    # plain call only (the front-end prep is listed apart): fetch x2, write x1,
    # each chain dispatch the mean of its two samples, two chain dispatches per call
    want = (2 * (1 + 1000 + 900 + 2 * 3000) + (1 + 300 + 200 + 2 * 100)) * 1024
    assert res["bytes_per_call"] == pytest.approx(want)
    assert [r[0][0] for r in res["others"]] == ["kda::prep_kernel<128, unsigned short, true, false>"]
    text = P.render(res, 256, ["cmd"], 1000)
    assert "| 2 | " in text   # the chain's dispatches per call


def test_traffic_record_follows_the_sources(tmp_path):
    f, w = str(tmp_path / "f"), str(tmp_path / "w")
    write_counters(f, [(ABS, "FETCH_SIZE", 1024), (PLAN, "FETCH_SIZE", 1), (PREP, "FETCH_SIZE", 1, 32 * 256 * 128),
                       (CHAIN, "FETCH_SIZE", 1)])
    write_counters(w, [(ABS, "WRITE_SIZE", 1024), (PLAN, "WRITE_SIZE", 1), (PREP, "WRITE_SIZE", 1, 32 * 256 * 128),
                       (CHAIN, "WRITE_SIZE", 1)])
    text = P.render(P.summarize(f, w, 1, P.PREFILL_8K), 1, ["cmd"], 1000)
    out = tmp_path / "t.md"
    out.write_text(text)
    rec = P.read_record(str(out))
    assert rec is not None and rec["source_digest"] == P.source_digest()
    stale = text.replace(P.source_digest(), "0" * 16)
    out.write_text(stale)
    assert P.read_record(str(out)) is None
    assert P.read_record(str(tmp_path / "missing.md")) is None


def test_mfma_busy_uses_one_xcd_of_active_cycles(tmp_path):
    d = str(tmp_path / "m")
    # 16 busy cycles per MFMA summed over the SIMDs; GRBM_GUI_ACTIVE summed
    # over 8 XCDs: 1000 cycles each
    busy = 0.5 * 1000 * P.SIMD_NUM
    write_counters(d, [(CHAIN, "SQ_VALU_MFMA_BUSY_CYCLES", busy), (CHAIN, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 2e6),
                       (CHAIN, "GRBM_GUI_ACTIVE", 8 * 1000),
                       ("void (anonymous namespace)::mfma_loop<1>(float*, int)", "SQ_VALU_MFMA_BUSY_CYCLES",
                        1000 * P.SIMD_NUM),
                       ("void (anonymous namespace)::mfma_loop<1>(float*, int)", "SQ_INSTS_VALU_MFMA_MOPS_BF16", 0),
                       ("void (anonymous namespace)::mfma_loop<1>(float*, int)", "GRBM_GUI_ACTIVE", 8000)])
    rows = {r[0]: r for r in P.mfma_summary(d)}
    assert rows["kda::chain_kernel<128, unsigned short, 1, false>"][3] == pytest.approx(50.0)
    assert rows["kda::chain_kernel<128, unsigned short, 1, false>"][4] == pytest.approx(2e6 * 512 / 1e9)
    assert rows["mfma_loop<1> (reference loop)"][3] == pytest.approx(100.0)


def test_prefill_grids_follow_the_shape():
    # one sequence of 4096 blocks at 32 heads: windows of about 1 GiB of
    # records (697 blocks at most), evened out: 5 x 683 + 681
    assert P.prefill_windows(1, 32, 4096) == [683] * 5 + [681]
    assert P.prefill_windows(1, 32, 256) == [256]
    assert P.prefill_windows(16, 32, 2756) == [2756]
    long = dict(P.WORKLOADS["prefill"][0])
    assert long[("kda::prep_kernel<128, unsigned short, false, false>", 32 * 683 * 128)] == 5
    assert long[("kda::prep_kernel<128, unsigned short, false, false>", 32 * 681 * 128)] == 1
    assert long[("kda::chain_kernel<128, unsigned short, 1, false>", 256 * 448)] == 6
    assert long[("kda::plan_kernel", 1024)] == 1
    short = dict(P.WORKLOADS["prefill_8k"][0])
    assert short[("kda::prep_kernel<128, unsigned short, false, false>", 32 * 256 * 128)] == 1
    assert short[("kda::chain_kernel<128, unsigned short, 1, false>", 256 * 448)] == 1
    # 16 sequences x 32 heads: 512 units (4096 slices, more than the CUs), 64
    # groups of 8 units x 4 two-slice workgroups of 512 threads
    assert dict(P.prefill_kernels(32, 2756, 512))[("kda::chain_kernel<128, unsigned short, 2, false>", 2048 * 512)] == 1


def test_kernel_key_keeps_template_arguments():
    assert P.kernel_key(CHAIN) == "kda::chain_kernel<128, unsigned short, 1, false>"
    assert P.kernel_key(PLAN) == "kda::plan_kernel"


def test_digest_ignores_comments_but_not_code():
    code = "int f(int a) {  // add one\n  return a + 1; /* done */\n}\n"
    assert P._code_only(code) == P._code_only("int f(int a) {\n return a + 1;\n}")
    assert P._code_only(code) != P._code_only(code.replace("a + 1", "a + 2"))


def test_memory_pipe_summary_per_cu_and_per_request(tmp_path):
    """Two passes of one chain dispatch: latency = latency sum / requests,
    shares = per-CU stall cycles / the active cycles of one XCD, hit rate from
    the L2 hit and miss counts; a kernel with next to no requests is left out."""
    def write(d, rows):
        os.makedirs(d, exist_ok=True)
        with open(os.path.join(d, "kda_counter_collection.csv"), "w", newline="") as fh:
            w = csv.DictWriter(fh, FIELDS)
            w.writeheader()
            for disp, k, c, v in rows:
                w.writerow({"Dispatch_Id": disp, "Kernel_Name": k, "Grid_Size": grid_of(k),
                            "Counter_Name": c, "Counter_Value": v})
    cyc = 1000.0                                   # per XCD; the CSV holds the sum over 8
    a, b = str(tmp_path / "a"), str(tmp_path / "b")
    write(a, [(1, CHAIN, "GRBM_GUI_ACTIVE", 8 * cyc),
              (1, CHAIN, "TCP_TCC_READ_REQ_sum", 256 * 400),
              (1, CHAIN, "TCP_TCC_READ_REQ_LATENCY_sum", 256 * 400 * 300),
              (1, CHAIN, "TCP_PENDING_STALL_CYCLES_sum", 256 * 0.5 * cyc),
              (2, PLAN, "GRBM_GUI_ACTIVE", 8 * cyc),
              (2, PLAN, "TCP_TCC_READ_REQ_sum", 3),
              (2, PLAN, "TCP_TCC_READ_REQ_LATENCY_sum", 900),
              (2, PLAN, "TCP_PENDING_STALL_CYCLES_sum", 0)])
    write(b, [(1, CHAIN, "GRBM_GUI_ACTIVE", 8 * cyc),
              (1, CHAIN, "TA_ADDR_STALLED_BY_TC_CYCLES_sum", 256 * 0.25 * cyc),
              (1, CHAIN, "TCC_HIT_sum", 870), (1, CHAIN, "TCC_MISS_sum", 130),
              (2, PLAN, "GRBM_GUI_ACTIVE", 8 * cyc),
              (2, PLAN, "TA_ADDR_STALLED_BY_TC_CYCLES_sum", 0),
              (2, PLAN, "TCC_HIT_sum", 1), (2, PLAN, "TCC_MISS_sum", 1)])
    rows = P.pipe_summary([a, b])
    assert len(rows) == 1
    k, n, cycles, req, lat, pend, tas, hit = rows[0]
    assert k == P.kernel_key(CHAIN) and n == 1
    assert cycles == pytest.approx(cyc) and req == pytest.approx(400)
    assert lat == pytest.approx(300) and pend == pytest.approx(50) and tas == pytest.approx(25)
    assert hit == pytest.approx(87)
