"""Build the fp64 CPU oracle (test infrastructure only) with gcc.

Only the tests, the smoke check and the benchmark's CPU-baseline leg use the
library this writes; the product path never loads it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "attention.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(src=SRC, out=LIB, extra_flags=()):
    """Compile `src` into the shared library `out`; returns `out`."""
    cmd = ["gcc", "-O2", "-std=c99", "-D_POSIX_C_SOURCE=200809L", "-shared", "-fPIC",
           "-Wall", "-Wextra", "-Werror", *extra_flags, "-o", out, src, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
