"""CPU test of the LDS tile layout: builds tests/host/lds_layout_check.cpp
against the kernels' own header (host code only, no GPU) and runs it."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_swizzle_is_a_permutation_and_bank_conflict_free(tmp_path):
    exe = tmp_path / "lds_layout_check"
    src = os.path.join(ROOT, "tests", "host", "lds_layout_check.cpp")
    build = subprocess.run(
        [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-std=c++17",
         "-I", os.path.join(ROOT, "exact_io_aware_28_amd", "csrc"),
         "-I", os.path.join(ROOT, "include"), src, "-o", str(exe)],
        capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-2000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True)
    assert run.returncode == 0, run.stdout
    assert run.stdout.strip().endswith("OK")
    assert run.stdout.count("conflicts 0, tr_b16 conflicts 0") == 4
    assert run.stdout.count("K b128 conflicts 0, V^T b128 conflicts 0") == 4
