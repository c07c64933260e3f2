"""Build the CPU oracle (plain C) into oracle/liboracle.so with gcc.

Test infrastructure only.  Flags keep IEEE semantics: no fast-math, no FMA
contraction, SSE arithmetic (FLT_EVAL_METHOD 0 on x86-64), so the one rounded
step of the method (AMCT's fp32 quotient) is a single correctly rounded
binary32 division.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mxfp4_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
          "-ffp-contract=off", "-fno-finite-math-only", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile the oracle; returns the path of the shared library."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force="--lazy" not in sys.argv))
