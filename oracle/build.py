"""Builds the CPU oracle (test infrastructure) into oracle/liboracle.so with gcc.

Plain single-threaded C11, -O2 -ffp-contract=off -fno-fast-math on x86-64 SSE2, so every
float and double operation is one IEEE-754 round-to-nearest-even operation.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")
SOURCES = ["oracle.c", "ziggurat.c"]


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
        "-Wall", "-Wextra", "-Wno-unused-parameter",
        "-o", LIB + ".tmp",
    ] + [os.path.join(HERE, s) for s in SOURCES] + ["-lquadmath", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
