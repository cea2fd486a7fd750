"""Compile the C oracle into a shared library (test infrastructure only).

The oracle is built with plain gcc, no FMA contraction and no fast-math, so
every double operation in oracle.c is one IEEE operation.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra"]


def build(source=SOURCE, out=LIBRARY, werror=True):
    """Compile `source` (default: oracle.c) to `out`; return the library path."""
    tmp = out + ".tmp"
    flags = CFLAGS + (["-Werror"] if werror else [])
    subprocess.run(["gcc", *flags, source, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
