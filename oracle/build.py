"""Compile the fp64 CPU oracle (test infrastructure) into oracle/liboracle.so."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "iabn_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def compile_source(src: str, out: str, verbose: bool = False) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c99", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Always recompiles; returns the library path."""
    return compile_source(SRC, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
