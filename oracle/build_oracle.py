"""Build the CPU oracle (oracle/liboracle.so) with gcc.

Test infrastructure: the oracle is compiled with IEEE-faithful flags (no
-ffast-math, no floating-point contraction) so its binary32 adds are exactly
the round-to-nearest-even additions it states.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

FLAGS = [
    "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror",
    "-fno-fast-math", "-ffp-contract=off", "-fno-unsafe-math-optimizations",
    "-fopenmp", "-fPIC", "-shared",
]


def build(verbose=False, src=SRC, out=LIB, extra=()):
    """Compile `src` into `out`; returns the output path."""
    tmp = out + ".tmp"
    cmd = ["gcc", *FLAGS, *extra, src, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
