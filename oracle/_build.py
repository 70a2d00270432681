"""Builds the CPU oracle (plain C, gcc, OpenMP) into oracle/liboracle.so.

Test infrastructure: the oracle is built here for the tests, the smoke check and
the benchmark's CPU baseline; the product library never links or loads it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fusednorm_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# -ffp-contract=off: no fused multiply-adds, so each fp32 / fp64 operation in the
# source is one correctly rounded IEEE operation. No fast-math.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-Wall",
          "-Wextra", "-Wno-unused-parameter"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def is_stale() -> bool:
    return not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC)


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
