"""Build libh2o.so in-tree with hipcc for gfx950, and its debug build.

Usage: python -m h2o_kv_cache_sdpa_amd.build  (or __graft_entry__.build()).
Objects go to h2o_kv_cache_sdpa_amd/_build/, the library to
h2o_kv_cache_sdpa_amd/libh2o.so.

The debug build (build_debug, also run by the module's main) compiles every
source with H2O_DEBUG (device-side index checks that trap instead of writing
outside a buffer) into libh2o_debug.so, and links abi_asan: the host code
of the ABI layer under AddressSanitizer, driven by abi_asan_main.cpp through
every entry point's validation paths (no GPU needed).  Its objects go to
h2o_kv_cache_sdpa_amd/_build_debug/.
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
DEBUG_BUILD = os.path.join(PKG, "_build_debug")
DEBUG_LIB = os.path.join(PKG, "libh2o_debug.so")
ASAN_EXE = os.path.join(DEBUG_BUILD, "abi_asan")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ROCM_LIB = "/opt/rocm/lib"

SOURCES = ["h2o_abi.cpp", "profile.cpp", "attn_simple.hip", "attn_mfma.hip", "attn_native.hip", "attn_quant.hip", "attn_short.hip", "attn_bwd.hip", "attn_bwd_dq.hip", "evict.hip", "kvwrite.hip"]

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


# Debug build: device index checks on, host debug info.
DEBUG_FLAGS = ["-DH2O_DEBUG", "-g"]
# Host code of the ABI layer under AddressSanitizer (host pass only: the
# device code of these files is not instrumented).
ASAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
ASAN_SOURCES = ["h2o_abi.cpp", "profile.cpp"]


def _run(cmd, what):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{what} failed:\n{r.stdout}\n{r.stderr}")


def _compile(src: str, outdir: str = BUILD, extra=(), tag: str = "") -> str:
    obj = os.path.join(outdir, tag + os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *EXTRA.get(src, []), *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    _run(cmd, f"hipcc for {src}")
    return obj


def _link_shared(objs, lib):
    tmp = lib + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], "link")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    _link_shared(objs, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def build_debug(verbose: bool = False) -> str:
    """libh2o_debug.so (device index checks) and the host ASan checker abi_asan."""
    os.makedirs(DEBUG_BUILD, exist_ok=True)
    jobs = [(s, DEBUG_BUILD, DEBUG_FLAGS, "") for s in SOURCES]
    jobs += [(s, DEBUG_BUILD, DEBUG_FLAGS + ASAN_HOST, "asan_") for s in ASAN_SOURCES]
    with ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    n = len(SOURCES)
    _link_shared(objs[:n], DEBUG_LIB)
    # the checker: plain host C++ under ASan, linked with the ASan objects of
    # the ABI layer and the debug objects of the kernels
    main_obj = os.path.join(DEBUG_BUILD, "abi_asan_main.o")
    _run(["g++", "-std=c++17", "-g", "-fsanitize=address", "-fno-omit-frame-pointer", "-c",
          os.path.join(CSRC, "abi_asan_main.cpp"), "-o", main_obj], "g++ abi_asan_main.cpp")
    kernel_objs = [o for s, o in zip(SOURCES, objs[:n]) if s not in ASAN_SOURCES]
    _run(["g++", "-fsanitize=address", main_obj, *objs[n:], *kernel_objs, f"-L{ROCM_LIB}", "-lamdhip64",
          f"-Wl,-rpath,{ROCM_LIB}", "-o", ASAN_EXE], "link abi_asan")
    if verbose:
        print(f"built {DEBUG_LIB} and {ASAN_EXE}")
    return DEBUG_LIB


if __name__ == "__main__":
    build(verbose=True)
    build_debug(verbose=True)
    sys.exit(0)
