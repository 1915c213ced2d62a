"""Compile the C oracle into ``oracle/liboracle.so`` with gcc.

TEST INFRASTRUCTURE ONLY: the library this builds is loaded by the test
suite, the smoke check and the benchmark's CPU-baseline leg, never by the
GPU library or its Python binding.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kvoracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    """Always recompiles; returns the path of the shared library."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-fno-fast-math", "-ffp-contract=off", "-D_GNU_SOURCE",
           SRC, "-o", LIB + ".tmp", "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
