"""Compile the C oracle into oracle/libhd_oracle.so with gcc.

TEST INFRASTRUCTURE ONLY: the oracle is the checker, not the product.
Run as ``python oracle/build.py`` or call :func:`build`.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "hd_oracle.c")
LIB = os.path.join(HERE, "libhd_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
