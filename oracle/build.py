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
# KVD_ORACLE_LIB selects another build of the same source (the sanitised
# one, for the sanitizer tier of the CPU tests)
LIB = os.environ.get("KVD_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")
SAN_LIB = os.path.join(HERE, "liboracle_san.so")


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Always recompiles; returns the path of the shared library.  With
    sanitize, an AddressSanitizer + UndefinedBehaviorSanitizer build (any
    report aborts) goes to liboracle_san.so; it needs libasan preloaded."""
    out = SAN_LIB if sanitize else LIB
    opt = (["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
            "-fno-sanitize-recover=all"] if sanitize else ["-O2"])
    cmd = ["gcc", *opt, "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-fno-fast-math", "-ffp-contract=off", "-D_GNU_SOURCE",
           SRC, "-o", out + ".tmp", "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv)
