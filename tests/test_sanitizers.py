"""The CPU test suites again, with AddressSanitizer and UndefinedBehaviorSanitizer
builds of the native code they run (each in a subprocess with the matching ASan
runtime preloaded; leak checking is off, since the Python interpreter itself is
not instrumented):

  - the C oracle built by gcc with -fsanitize=address,undefined, under the
    oracle's pins, planted mistakes, gate variants and front end;
  - the host side of libkda (kda_api.hip: validation, sizing, the host copy of
    cu_seqlens) built by hipcc with the sanitizers on the host pass only and
    linked with the uninstrumented kernel objects, under the C-ABI and binding
    tests (which never launch a kernel).
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ASAN_OPTIONS = "detect_leaks=0:alloc_dealloc_mismatch=0:abort_on_error=1"


def _run(args, env, timeout=900):
    return subprocess.run([sys.executable, *args], env=env, cwd=ROOT, capture_output=True, text=True,
                          timeout=timeout)


def _check(r):
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_and_ubsan():
    from oracle import build as oracle_build
    lib = oracle_build.build(sanitize=True)
    runtime = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    assert os.path.isabs(runtime) and os.path.exists(runtime)
    env = dict(os.environ, LD_PRELOAD=runtime, ASAN_OPTIONS=ASAN_OPTIONS, KDA_ORACLE_LIB=lib, OMP_NUM_THREADS="4")
    r = _run(["-c", "from oracle import reference; print(reference.lib()._name)"], env, timeout=120)
    _check(r)
    assert r.stdout.strip() == lib
    _check(_run(["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                 "tests/test_oracle_pins.py", "tests/test_oracle_mutations.py", "tests/test_oracle_variants.py",
                 "tests/test_oracle_frontend.py"], env))


def test_c_abi_host_side_under_asan_and_ubsan():
    from gated_delta_rule_109_amd import build
    if not os.path.exists(build.HIPCC):
        pytest.skip("needs hipcc")
    lib = build.build_host_sanitized()
    env = dict(os.environ, LD_PRELOAD=build.san_runtime(), ASAN_OPTIONS=ASAN_OPTIONS, KDA_LIB=lib)
    r = _run(["-c", "from gated_delta_rule_109_amd import kda; print(kda.lib()._name)"], env, timeout=120)
    _check(r)
    assert r.stdout.strip() == lib
    _check(_run(["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                 "tests/test_abi.py", "tests/test_binding.py"], env))
