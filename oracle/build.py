"""Compile the C oracle into oracle/libgqa_oracle.so with gcc.

Test infrastructure: the oracle is only ever loaded by the test suite, the
smoke check and the benchmark's CPU-baseline leg.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gqa_oracle.c")
LIB = os.path.join(HERE, "libgqa_oracle.so")


def build(verbose: bool = False) -> str:
    """Always recompiles (plain -O2, IEEE semantics: no -ffast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           "-fno-fast-math", "-ffp-contract=off", SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
