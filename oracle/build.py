"""Compile the CPU oracle (``oracle/pao.c``) into ``oracle/liboracle.so``.

Test infrastructure only: it compiles the reference the tests compare
against; nothing in the product library uses it.  Plain ``gcc -std=c11 -O2`` (no fast-math, so float64 sums
keep their written order) with OpenMP for the outer (sequence, head) loops.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "pao.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-Werror", SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
