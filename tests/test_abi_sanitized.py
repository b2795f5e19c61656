"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/sanitize_abi.cpp calls every entry point of include/m2rnn.h with
arguments that fail validation (negative or unsupported sizes, bad dtype,
NULL or misaligned pointers, missing or short workspaces), which the library
rejects before any HIP call, and queries every workspace size at the extremes
of int.  This test builds it together with the library sources, host code
under -fsanitize=address,undefined with no recovery (the device code is
compiled as usual and never launched), and runs it without a GPU.  Each call
must return its documented status with a message, and no size computation may
overflow."""
import glob
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="hipcc not available")
def test_abi_host_code_clean_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "sanitize_abi")
    srcs = sorted(glob.glob(os.path.join(ROOT, "non_linear_matrix_amd", "csrc", "*.hip")))
    cmd = [HIPCC, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "non_linear_matrix_amd", "csrc"),
           *srcs, os.path.join(HERE, "sanitize_abi.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert build.returncode == 0, build.stdout + build.stderr
    # leak checking is off: the HIP runtime's own allocations outlive main
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    report = run.stdout + run.stderr
    assert run.returncode == 0, report
    assert "runtime error" not in report and "AddressSanitizer" not in report, report
    assert "all calls clean" in run.stdout
