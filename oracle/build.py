"""Build the oracle's shared library (plain C, host compiler only).

The oracle is test infrastructure: only the tests, the smoke check and the
benchmark's CPU-baseline leg load it.

Two builds:
 * liboracle.so       -O2 with OpenMP (the GEMM routines spread output rows
                      over the host cores; every entry is still one sequential
                      loop, so results do not depend on the thread count);
 * liboracle_san.so   the same source under AddressSanitizer and
                      UndefinedBehaviorSanitizer, without OpenMP, loaded only
                      by the sanitizer test (in a child process that preloads
                      the ASan runtime).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")
SAN_LIB = os.path.join(HERE, "liboracle_san.so")
SRC = os.path.join(HERE, "mx_oracle.c")
HDR = os.path.join(HERE, "mx_oracle.h")

# -ffp-contract=off: the NVFP4 sequence is one IEEE fp32 rounding per step.
CFLAGS = ["-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
          "-fno-fast-math", "-fPIC", "-shared"]
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined", "-Wno-unknown-pragmas"]


def _stale(lib):
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    return t < os.path.getmtime(SRC) or t < os.path.getmtime(HDR)


def build(force=True):
    """Compile mx_oracle.c into liboracle.so next to it; returns the path."""
    if not force and not _stale(LIB):
        return LIB
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, "-fopenmp", SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def build_sanitized(force=True):
    """Compile the ASan + UBSan variant, liboracle_san.so; returns the path."""
    if not force and not _stale(SAN_LIB):
        return SAN_LIB
    tmp = SAN_LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, *SAN_FLAGS, SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    print(build(force="--if-stale" not in sys.argv))
    if "--sanitize" in sys.argv:
        print(build_sanitized())
