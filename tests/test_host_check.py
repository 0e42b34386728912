"""CPU debug build of the library's host side (tests/host_check/hs_host_check.hip):
problem validation, the packed-document block table, the decode split plan,
the gradient workspace layout and the index arithmetic shared with the
kernels, built with AddressSanitizer and UndefinedBehaviorSanitizer (array
bounds included) on the host only, checked against brute force and run with
stub launchers that check every workspace pointer the entry points carve.
No GPU is needed."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host_check", "hs_host_check.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def test_host_planners_under_sanitizers(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    exe = str(tmp_path / "hs_host_check")
    flags = ["-O1", "-g", "-std=c++17", "--offload-arch=gfx950",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address",
             "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all",
             "-I", os.path.join(ROOT, "include"),
             "-I", os.path.join(ROOT, "block_sparse_mqa_amd", "csrc")]
    build = subprocess.run([HIPCC, *flags, SRC, "-o", exe], capture_output=True, text=True,
                           timeout=900)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    for seed in ("1", "2"):
        run = subprocess.run([exe, "600", seed], capture_output=True, text=True, timeout=600,
                             env=env)
        assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-4000:])
        assert "all checks passed" in run.stdout, run.stdout[-2000:]
