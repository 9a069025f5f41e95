"""Compile the HIP sources under csrc/ into libattn.so (gfx950), in-tree.

Run as ``python -m exact_blockwise_attention_attn_amd._build`` or call
``build_library()``.  Every call recompiles.  Object files go to ``_build/`` next
to this file; the library lands beside this file as ``libattn.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libattn.so")
ARCH = "gfx950"

SOURCES = ["attn_api.cpp", "attn_fwd_bf16.hip", "attn_fwd_bf16_d64.hip", "attn_fwd_f32.hip", "attn_bwd_bf16.hip",
           "attn_decode_bf16.hip", "attn_noalloc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU forms stay disabled in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wno-unused-command-line-argument",
]


# Per-source flags.  The bf16 kernel never produces or consumes NaN (masked scores
# are -inf, every row has an allowed key), so NaN-quieting canonicalisations can go
# and the row maximum maps onto v_max3_f32.
# attn_bwd_bf16.hip: matrix-instruction accumulators in VGPRs.  Left to choose, the
# compiler puts the dQ kernel's score and dP accumulators in AGPRs and copies all 32
# of them to VGPRs on every key tile for the vector work (352 copies in the kernel);
# with this form it uses 200 VGPRs, no AGPRs and no copies, at the same occupancy.
# attn_fwd_bf16_d64.hip (the dense d = 64 forward kernels): the same form lifts their
# occupancy; the d = 128 forward kernels stay in the default form.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
PER_SOURCE = {"attn_fwd_bf16.hip": ["-fno-honor-nans"],
              "attn_fwd_bf16_d64.hip": ["-fno-honor-nans", *VGPR_FORM],
              "attn_bwd_bf16.hip": ["-fno-honor-nans", *VGPR_FORM]}


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *PER_SOURCE.get(src, []), *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build_library(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile every source and link libattn.so; returns the library path."""
    os.makedirs(OBJ, exist_ok=True)
    extra = list(extra or [])
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build_library(verbose=True, extra=sys.argv[1:])
