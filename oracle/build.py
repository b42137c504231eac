"""Builds the fp64 CPU oracle (``liboracle_attnres.so``) with gcc.

TEST INFRASTRUCTURE ONLY: the oracle checks the GPU library; it is never part
of the product path.  Plain ``-O2`` with no fast-math, so every step stays
IEEE double in the order the source writes it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "attnres_oracle.c")
LIB = os.path.join(HERE, "liboracle_attnres.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-fno-fast-math",
           "-fPIC", "-shared", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def ensure_built() -> str:
    """Builds the oracle if the library is absent or older than its source."""
    if (not os.path.exists(LIB)
            or os.path.getmtime(LIB) < os.path.getmtime(SRC)):
        build()
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
