"""Builds libgdntree.so (the gfx950 kernels and the C ABI) with hipcc.

    python __graft_entry__.py      (or __graft_entry__.build())
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgdntree.so")
SOURCES = ["gdntree_api.hip", "build_tree.hip", "verify_tree.hip", "accept_commit.hip", "commit_build.hip",
           "shared_budget.hip", "markov_edges.hip"]
# the benchmark's streaming probe, in a library of its own (not part of the path's ABI)
PROBE_SOURCES = ["stream_probe.hip"]
PROBE_LIB = os.path.join(HERE, "libgdntree_probe.so")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fvisibility=hidden",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    _build_one(PROBE_LIB, PROBE_SOURCES, verbose, extra)
    return _build_one(LIB, SOURCES, verbose, extra)


def _build_one(lib: str, sources: list[str], verbose: bool, extra: list[str] | None) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = lib + ".tmp"
    cmd = [hipcc, *FLAGS, *(extra or []), *[os.path.join(CSRC, s) for s in sources], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(x for x in res.stderr.splitlines() if noise not in x)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
