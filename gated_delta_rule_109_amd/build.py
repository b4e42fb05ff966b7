"""Build libkda.so (the HIP library behind include/kda.h) in-tree for gfx950,
and libkda_peak.so, a measurement helper (a bf16 MFMA loop that bench.py times
as the measured matrix rate; not part of the KDA library).

Each .hip source is compiled with hipcc for gfx950 only, then linked into
gated_delta_rule_109_amd/libkda.so. Packed-fp32 VALU instructions are turned
off for the device code (-packed-fp32-ops); hipcc's host pass warns that it
does not know that feature, which is harmless.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libkda.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["kda_api.hip", "kda_decode.hip", "kda_prefill.hip"]
PEAK_SOURCE = os.path.join(CSRC, "measure", "peak_mfma.hip")
PEAK_LIB = os.path.join(HERE, "libkda_peak.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC] + DEVICE_FLAGS


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        _run([HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    tmp = PEAK_LIB + ".tmp"
    _run([HIPCC, *CFLAGS, "-shared", PEAK_SOURCE, "-o", tmp], verbose)
    os.replace(tmp, PEAK_LIB)
    return LIB


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer build of the C ABI
# (argument validation, sizing, the plan's host arithmetic): kda_api.hip with
# the host pass instrumented and the device code untouched, linked with the
# uninstrumented kernel objects of build() into libkda_san.so. Load it with
# clang's ASan runtime preloaded (SAN_RUNTIME); for CPU tests of the C ABI only.
SAN_LIB = os.path.join(HERE, "libkda_san.so")
SAN_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-Xarch_host", "-fno-sanitize-recover=all", "-g"]
SAN_RUNTIME = os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib", "clang")


def san_runtime() -> str:
    """clang's shared ASan runtime (the one hipcc's host pass instruments for)."""
    import glob
    hits = sorted(glob.glob(os.path.join(SAN_RUNTIME, "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise FileNotFoundError("libclang_rt.asan-x86_64.so not found under " + SAN_RUNTIME)
    return hits[-1]


def build_host_sanitized(verbose: bool = False) -> str:
    objs = [os.path.join(BUILD_DIR, s.replace(".hip", ".o")) for s in SOURCES if s != "kda_api.hip"]
    for o in objs:
        if not os.path.exists(o):
            build(verbose)
            break
    san_obj = os.path.join(BUILD_DIR, "kda_api_san.o")
    _run([HIPCC, *CFLAGS, *SAN_HOST_FLAGS, "-c", os.path.join(CSRC, "kda_api.hip"), "-o", san_obj], verbose)
    clangxx = os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "bin", "clang++")
    link = [clangxx, "-shared", "-shared-libsan", "-fsanitize=address,undefined", "-o", SAN_LIB + ".tmp",
            san_obj, *objs, "-L" + os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "lib"), "-lamdhip64"]
    _run(link, verbose)
    os.replace(SAN_LIB + ".tmp", SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    if "--host-sanitized" in sys.argv:
        print(build_host_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
