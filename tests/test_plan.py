"""CPU check of the prefill plan's index arithmetic (csrc/kda_plan.h).

The plan and chain kernels derive every table from the device copy of
cu_seqlens; the launches are sized from the host copy. plan_check.cpp runs the
same header functions on the CPU over seeded host / device pairs and record
windows, and checks that equal copies give the exact tables (and windows that
cover every sequence once, with one carried state per window edge) and that
copies that differ never reach a record, row, checkpoint slot or table entry
outside what the host copy sized.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_plan_index_arithmetic(tmp_path):
    exe = str(tmp_path / "plan_check")
    src = os.path.join(HERE, "plan_check.cpp")
    subprocess.run(["g++", "-O1", "-std=c++17", "-Wall", "-Wextra", "-Werror", "-fsanitize=undefined",
                    "-fno-sanitize-recover=all", "-o", exe, src], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.startswith("ok ")
