"""Compile the CPU oracle (plain C) into oracle/liboracle.so with gcc.

Test infrastructure: the oracle is loaded only by the test suite, the smoke
check and the CPU-baseline leg of the benchmark.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# No fast-math: the oracle's fp32 divisions must be correctly rounded and its
# fp64 sums evaluated in the order written.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra", "-Werror"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
