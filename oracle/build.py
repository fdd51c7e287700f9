"""Compile the fp64 reference (kla_oracle.c) into oracle/libkla_oracle.so.

Test infrastructure: the library is loaded only by the tests, the smoke
check and the CPU-baseline leg of the benchmark.  Plain gcc, -O2, OpenMP,
no fast-math (the reference must keep IEEE double semantics).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kla_oracle.c")
LIB = os.path.join(HERE, "libkla_oracle.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-fno-fast-math", "-ffp-contract=off",
           SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
