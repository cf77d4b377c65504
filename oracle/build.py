"""Build the oracle's shared library (plain C, host compiler only).

The oracle is test infrastructure: only the tests, the smoke check and the
benchmark's CPU-baseline leg load it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")
SRC = os.path.join(HERE, "mx_oracle.c")

# -ffp-contract=off: the NVFP4 sequence is one IEEE fp32 rounding per step.
CFLAGS = ["-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
          "-fno-fast-math", "-fPIC", "-shared"]


def build(force=True):
    """Compile mx_oracle.c into liboracle.so next to it; returns the path."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force="--if-stale" not in sys.argv))
