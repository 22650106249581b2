"""Build the gfx950 shared library ``libcp_attn.so`` in-tree with hipcc.

Usage: ``python -m long_sequence_causal_cp_amd.build`` (or ``build()``).
Cross-compiles without a GPU.  Packed-fp32 VALU instructions are disabled
(``-packed-fp32-ops``); every kernel is compiled for gfx950 only.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libcp_attn.so")

SOURCES = ["cp_attn_kernels.hip", "cp_attn_bwd.hip", "cp_attn_fp8.hip", "cp_ring_plan.cpp", "cp_attn_api.cpp",
           "cp_attn_noalloc.hip"]
CEILING_SRC = os.path.join(CSRC, "mfma_ceiling.hip")  # measurement tool, its own executable
CEILING_BIN = os.path.join(HERE, "mfma_ceiling")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run_hipcc(args, out: str, verbose: bool) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), *args, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Build libcp_attn.so and the mfma_ceiling measurement tool; return the library path."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    _run_hipcc([*FLAGS, "-I", os.path.join(ROOT, "include"), *srcs], LIB, verbose)
    exe_flags = [f for f in FLAGS if f not in ("-fPIC", "-shared")]
    _run_hipcc([*exe_flags, CEILING_SRC], CEILING_BIN, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
