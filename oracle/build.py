"""Build the fp64 CPU oracle (plain C) into oracle/libm2rnn_ref.so with gcc.

Test infrastructure only: the oracle serves the test suite, the package smoke
check and the benchmark's CPU-baseline leg.  It is never part of the product
path.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "m2rnn_ref.c")
LIB = os.path.join(HERE, "libm2rnn_ref.so")


def build(src=SRC, out=LIB, extra_flags=()):
    """Compile `src` into the shared library `out`; returns `out`."""
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-D_POSIX_C_SOURCE=200809L", *extra_flags, "-o", out, src,
           "-lm", "-lpthread"]
    tmp = out + ".tmp"
    cmd[cmd.index(out)] = tmp
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
    sys.exit(0)
