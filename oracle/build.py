"""Compile the CPU oracle (plain C, gcc) into oracle/libqblk_oracle.so.

Test infrastructure: the oracle is the checker, never part of the product.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qblk_oracle.c")
LIB = os.path.join(HERE, "libqblk_oracle.so")

# IEEE binary32 everywhere: SSE arithmetic (x86-64 default), no contraction of
# a*b+c into a fused multiply-add, no fast-math, no excess precision.
CFLAGS = [
    "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
    "-fexcess-precision=standard", "-fno-strict-aliasing",
    "-Wall", "-Wextra", "-Werror", "-fPIC", "-shared",
]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
