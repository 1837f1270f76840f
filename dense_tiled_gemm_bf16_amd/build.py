"""Build libtgemm.so in-tree with hipcc for gfx950.

    python -m dense_tiled_gemm_bf16_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libtgemm.so")
SOURCES = [os.path.join(CSRC, "tgemm_kernels.hip"), os.path.join(CSRC, "tgemm_quant.hip"),
           os.path.join(CSRC, "tgemm_clock.hip"), os.path.join(CSRC, "tgemm_scratch.hip"),
           os.path.join(CSRC, "tgemm_abi.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-command-line-argument", "-fvisibility=hidden",
    # (Device helpers are unused in the host pass, which compiles no kernel bodies.)
    "-Wno-unneeded-internal-declaration",
    # No packed-fp32 VALU instructions (v_pk_*_f32) in device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False) -> str:
    cmd = [HIPCC, *FLAGS, "-o", LIB + ".tmp", *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that line.
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
