"""Build the C part of the CPU oracle (test infrastructure only).

Compiles oracle/q8.c with gcc into oracle/liboracle.so.  The flags keep every
binary32 operation separately rounded: no contraction into FMA, no fast-math,
no flush-to-zero.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")
SRC = os.path.join(HERE, "q8.c")
CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC"]


def build(verbose: bool = False) -> str:
    """Compile liboracle.so (always recompiles) and return its path."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
