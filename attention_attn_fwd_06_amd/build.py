"""Build the gfx950 attention library in-tree with hipcc.

    python -m attention_attn_fwd_06_amd.build

produces ``attention_attn_fwd_06_amd/libattn_mi355x.so`` from ``csrc/*.hip``.
"""
from __future__ import annotations

import os
import pathlib
import subprocess
import sys

PKG = pathlib.Path(__file__).resolve().parent
CSRC = PKG / "csrc"
LIB = PKG / "libattn_mi355x.so"
INCLUDE = PKG.parent / "include"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU ops stay disabled (hipcc -O3 would otherwise form them)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the prefill's fully unrolled step at head dim 256 (64 MFMA slots) is larger
    # than the default limit for `#pragma unroll`; left rolled, its register
    # arrays are indexed at run time and spill to scratch (2 KB per lane, 50x
    # slower).  The other kernels compile to the same code either way.
    "-mllvm", "-pragma-unroll-threshold=100000",
    "-Wall", "-Wno-unused-function",
]
SOURCES = ["attn_api.hip", "prefill_fwd.hip", "decode.hip"]


def build(verbose: bool = False) -> pathlib.Path:
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [HIPCC, *FLAGS, f"-I{INCLUDE}", *[str(CSRC / s) for s in SOURCES], "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
