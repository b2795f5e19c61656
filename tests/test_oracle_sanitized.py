"""The fp64 CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/sanitize_oracle.c drives every oracle entry point on odd sizes, with
and without each optional argument, on one, several and all host threads,
and with bad arguments; this test compiles it together with
oracle/m2rnn_ref.c with -fsanitize=address,undefined (no recovery) and runs
it.  Any out-of-bounds access, use after free, leak, signed overflow or other
undefined behaviour aborts the run with a sanitizer report."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE = os.path.join(os.path.dirname(HERE), "oracle")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_clean_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "sanitize_oracle")
    cmd = ["gcc", "-O1", "-g", "-std=c99", "-D_POSIX_C_SOURCE=200809L", "-Wall", "-Wextra",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-I", ORACLE, os.path.join(HERE, "sanitize_oracle.c"), os.path.join(ORACLE, "m2rnn_ref.c"),
           "-o", exe, "-lm", "-lpthread"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    # (a library the environment preloads may come before the ASan runtime)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    report = run.stdout + run.stderr
    assert run.returncode == 0, report
    assert "runtime error" not in report and "AddressSanitizer" not in report, report
    assert "all calls clean" in run.stdout
