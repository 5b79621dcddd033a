"""Build libkda.so (HIP, gfx950) in-tree with hipcc.

All device code is compiled for gfx950 only, with packed-fp32 instructions
disabled (hipcc is told `-target-feature -packed-fp32-ops`).  The library is
written next to this file as ``libkda.so``.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkda.so")
SOURCES = ["kda_api.hip", "kda_chunk.hip", "kda_decode.hip", "kda_merge.hip", "kda_backward.hip",
           "kda_check.hip", "kda_bwgrad.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(out: str = LIB, verbose: bool = False, extra=()) -> str:
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-function", *extra,
           "-I", os.path.join(HERE, "..", "include"),
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def build_stamps(verbose: bool = False) -> str:
    """The profiling variant, with the chunk kernel's phase timestamps
    (kda_debug_phase_stamps), as libkda_stamps.so beside libkda.so."""
    return build(os.path.join(HERE, "libkda_stamps.so"), verbose, extra=("-DKDA_PHASE_STAMPS",))


if __name__ == "__main__":
    if "--stamps" in sys.argv[1:]:
        print(build_stamps(verbose=True))
    else:
        print(build(verbose=True))
    sys.exit(0)
