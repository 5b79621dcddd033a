"""Build the fp64 KDA oracle (test infrastructure) as a shared library with gcc.

Plain C, -O2, no -ffast-math (the oracle must evaluate fp64 exactly as written),
OpenMP over independent heads.  ``mutant`` builds a planted-mistake variant into
another file for the oracle's own pin tests.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kda_oracle.c")
LIB = os.path.join(HERE, "libkda_oracle.so")


def build(out: str = LIB, mutant: int = 0, verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
           "-ffp-contract=off", f"-DKDA_ORACLE_MUTANT={int(mutant)}", SRC, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
