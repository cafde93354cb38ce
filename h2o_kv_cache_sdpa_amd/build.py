"""Build libh2o.so in-tree with hipcc for gfx950.

Usage: python -m h2o_kv_cache_sdpa_amd.build  (or __graft_entry__.build()).
Objects go to h2o_kv_cache_sdpa_amd/_build/, the library to
h2o_kv_cache_sdpa_amd/libh2o.so.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libh2o.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["h2o_abi.cpp", "profile.cpp", "attn_simple.hip", "attn_mfma.hip", "attn_native.hip", "attn_quant.hip", "attn_bwd.hip", "attn_bwd_dq.hip", "evict.hip", "kvwrite.hip"]

# Packed fp32 VALU forms are disabled: every fp32 operation is issued as a
# scalar-per-lane instruction.  No fast-math: the quantisers rely on IEEE
# division and round-to-nearest-even.
COMMON = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


# Per-source flags.  The dQ kernel runs one wavefront per SIMD with more than
# 256 registers; by default the S / dP results of its MFMAs land in
# accumulation registers and are copied out before every exponential.  The
# VGPR form of the MFMAs keeps them where the vector ALU reads them (measured
# faster for dQ, slower for the dK/dV kernel, which keeps the default).
EXTRA = {"attn_bwd_dq.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
