"""Build the CPU oracle (plain C, gcc) into oracle/liboracle.so.

Test infrastructure: the oracle is built so the tests, the smoke check and the
benchmark's CPU-baseline leg can load it. The GPU library never links it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")
SRC = os.path.join(HERE, "zs_oracle.c")

# -ffp-contract=off: no fused multiply-add, so every float operator rounds
# once. No -ffast-math (it would flush subnormals and reorder), no -march
# (no implicit FMA); x86-64 SSE arithmetic has no excess precision.
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
