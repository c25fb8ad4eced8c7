"""Build the CPU oracle library ``oracle/liboracle.so`` with gcc.

Test infrastructure: the flags make each C expression in ``oracle.c`` exactly
one IEEE-754 binary32 operation (no fast-math, no contraction into FMA, SSE
arithmetic rather than x87 excess precision).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = [
    "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off",
    "-mfpmath=sse", "-msse2", "-fPIC", "-shared", "-Wall", "-Wextra",
]


def build(verbose: bool = False) -> str:
    """Compile the oracle; returns the path of the shared library."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
