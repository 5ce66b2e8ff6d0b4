"""Build step for the CPU oracle (test infrastructure).

Compiles ``det_gemm_oracle.c`` with gcc into ``liboracle.so`` beside it:
strict IEEE fp32 (no fast-math, and no contraction into fused multiply-add
beyond the explicit fmaf of a leaf step) and OpenMP across output rows.
``-mfma`` lets fmaf compile to the x86-64 FMA3 instruction (every x86-64
server CPU of the last decade has it) instead of a library call.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "det_gemm_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-std=c99", "-O2", "-fno-fast-math", "-ffp-contract=off", "-mfma", "-fopenmp",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile the oracle library; returns its path."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force="--if-stale" not in sys.argv))
