"""Compile the plain-C oracle (test infrastructure only) with gcc.

``build()`` always recompiles ``oracle/ref_cpu.c`` into
``oracle/libssmoracle.so``.  Flags: -ffp-contract=off so that only explicit
fmaf() calls fuse, no fast-math, OpenMP for the row loop.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ref_cpu.c")
LIB = os.path.join(HERE, "libssmoracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-std=c11", "-Wall", "-shared", "-fPIC", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
