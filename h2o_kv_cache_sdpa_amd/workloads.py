"""Seeded synthetic inputs for the H2O chunk step.

This module only draws random numbers and rounds them to the storage precision
(fp32 or bf16, round to nearest even).  It holds none of the method's
arithmetic, imports neither the GPU library nor the oracle, and is the one
module both sides share.

Shapes and value distributions stand in for the workloads the pages describe:
Helmet sequences of 64K/128K tokens streamed through a Qwen3-4B-class layer with
8 KV heads of dimension 128 and a cache of 16K/32K slots, chunks of 1K/2K tokens
("Learning how to Forget", §3.3 and §4; the aimodeling article on the
KeysAndValues release).  No dataset or trained weight is used: queries, keys and
values are i.i.d. N(0, 1); a few "heavy hitter" keys are scaled by 4 so that
some slots draw much more attention than others.

Seeding: chunk ``step`` of workload ``cfg_id`` uses
``numpy.random.default_rng([cfg_id, step])``; a prefilled cache uses
``default_rng([cfg_id, PREFILL_STREAM])``.  Draw order: q, k, v, then the
heavy-hitter rows per (b, g) in row-major order.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

PREFILL_STREAM = 2**31 - 1


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    B: int
    Hq: int
    Hkv: int
    D: int
    C: int
    T: int
    n_fill: int          # chunk steps that fill an empty cache
    n_evict: int         # chunk steps that evict from a full cache
    dtype: str           # "f32" or "bf16": Q, K_new, V_new and the native cache
    cache_fmt: str       # "native", "int8" or "int4"
    hh_new: float = 0.0  # fraction of each chunk's keys scaled by 4, per (b, g)
    hh_cache: float = 0.0  # fraction of a prefilled cache's keys scaled by 4
    start_full: bool = False  # cache starts full (single evicting step)
    prior_hi: float = 0.0  # prefilled scores ~ U(0, prior_hi)

    @property
    def qg(self):
        return self.Hq // self.Hkv

    @property
    def steps(self):
        return self.n_fill + self.n_evict

    @property
    def tokens(self):
        return self.T * self.steps

    def scaled(self, **kw):
        """A copy with some sizes replaced (for tests at reduced size)."""
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    1: Workload("tiny_f32_stream", 1, B=1, Hq=4, Hkv=1, D=64, C=256, T=32,
                n_fill=8, n_evict=8, dtype="f32", cache_fmt="native"),
    2: Workload("bf16_single_step_16k", 2, B=1, Hq=32, Hkv=8, D=128, C=16384, T=1024,
                n_fill=0, n_evict=1, dtype="bf16", cache_fmt="native",
                hh_cache=0.02, start_full=True, prior_hi=50.0),
    3: Workload("bf16_stream_32k_t2048", 3, B=1, Hq=32, Hkv=8, D=128, C=32768, T=2048,
                n_fill=16, n_evict=48, dtype="bf16", cache_fmt="native", hh_new=0.02),
    4: Workload("int8_stream_16k_t1024", 4, B=1, Hq=32, Hkv=8, D=128, C=16384, T=1024,
                n_fill=16, n_evict=48, dtype="bf16", cache_fmt="int8"),
    5: Workload("int4_batch4_32k_t1024", 5, B=4, Hq=32, Hkv=8, D=128, C=32768, T=1024,
                n_fill=32, n_evict=96, dtype="bf16", cache_fmt="int4", hh_new=0.02),
}


# --------------------------------------------------------------------------
# storage rounding
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x):
    """float32 -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits):
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


@dataclass
class Stored:
    """A tensor in its storage format plus its exact values as float64."""
    raw: np.ndarray   # float32, or uint16 bf16 bit patterns
    f64: np.ndarray
    dtype: str

    @property
    def f32(self):
        return self.f64.astype(np.float32)


def to_storage(x64, dtype):
    x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return Stored(x32, x32.astype(np.float64), dtype)
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x32)
        return Stored(bits, bf16_bits_to_f32(bits).astype(np.float64), dtype)
    raise ValueError(dtype)


def _heavy_hitters(rng, x, frac):
    """Scale a fraction of rows (axis 2) by 4, chosen independently per (b, g)."""
    if frac <= 0:
        return x
    B, H, N = x.shape[:3]
    n_hh = int(round(frac * N))
    for b in range(B):
        for g in range(H):
            rows = rng.choice(N, size=n_hh, replace=False)
            x[b, g, rows, :] *= 4.0
    return x


# --------------------------------------------------------------------------
# generators
# --------------------------------------------------------------------------

def random_chunk(seed, B, Hq, Hkv, T, D, dtype, hh_frac=0.0, q_zero=False):
    """One chunk of queries and new keys/values: N(0,1), rounded to ``dtype``."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, T, D))
    k = rng.standard_normal((B, Hkv, T, D))
    v = rng.standard_normal((B, Hkv, T, D))
    k = _heavy_hitters(rng, k, hh_frac)
    if q_zero:
        q[:] = 0.0
    return dict(q=to_storage(q, dtype), k=to_storage(k, dtype), v=to_storage(v, dtype))


def chunk(w: Workload, step: int):
    return random_chunk([w.cfg_id, step], w.B, w.Hq, w.Hkv, w.T, w.D, w.dtype, w.hh_new)


def random_cache(seed, B, Hkv, C, D, n_occ, dtype, hh_frac=0.0, prior_hi=50.0):
    """A cache whose first n_occ slots hold N(0,1) keys/values, prior scores
    ~ U(0, prior_hi) as fp32, token_pos[j] = j; returns (k, v, scores_f32, token_pos, pos)."""
    rng = np.random.default_rng(seed)
    k = np.zeros((B, Hkv, C, D))
    v = np.zeros((B, Hkv, C, D))
    k[:, :, :n_occ] = rng.standard_normal((B, Hkv, n_occ, D))
    v[:, :, :n_occ] = rng.standard_normal((B, Hkv, n_occ, D))
    if n_occ:
        k[:, :, :n_occ] = _heavy_hitters(rng, k[:, :, :n_occ].copy(), hh_frac)
    scores = np.zeros((B, Hkv, C), np.float32)
    scores[:, :, :n_occ] = rng.uniform(0.0, prior_hi, size=(B, Hkv, n_occ)).astype(np.float32)
    token_pos = np.full((B, Hkv, C), -1, np.int32)
    token_pos[:, :, :n_occ] = np.arange(n_occ, dtype=np.int32)
    return to_storage(k, dtype), to_storage(v, dtype), scores, token_pos, n_occ


def prefilled_cache(w: Workload):
    return random_cache([w.cfg_id, PREFILL_STREAM], w.B, w.Hkv, w.C, w.D, w.C,
                        w.dtype, w.hh_cache, w.prior_hi)


def random_quant_cache(seed, B, Hkv, C, D, n_occ, fmt, prior_hi=50.0):
    """A quantised cache with random codes and fp16 scales (and zero points)
    in its first n_occ slots.  Returns a dict of raw arrays in storage format:
    k_codes, v_codes, k_scale, v_scale (fp16), k_zero, v_zero (fp16, int4 only),
    scores (fp32), token_pos (int32)."""
    rng = np.random.default_rng(seed)
    out = {}
    for name in ("k", "v"):
        if fmt == "int8":
            codes = np.zeros((B, Hkv, C, D), np.int8)
            codes[:, :, :n_occ] = rng.integers(-127, 128, size=(B, Hkv, n_occ, D), dtype=np.int8)
            scale = np.zeros((B, Hkv, C), np.float16)
            scale[:, :, :n_occ] = rng.uniform(0.004, 0.04, size=(B, Hkv, n_occ)).astype(np.float16)
            out[name + "_codes"], out[name + "_scale"] = codes, scale
        elif fmt == "int4":
            codes = np.zeros((B, Hkv, C, D // 2), np.uint8)
            codes[:, :, :n_occ] = rng.integers(0, 256, size=(B, Hkv, n_occ, D // 2), dtype=np.uint8)
            scale = np.zeros((B, Hkv, C), np.float16)
            scale[:, :, :n_occ] = rng.uniform(0.2, 0.6, size=(B, Hkv, n_occ)).astype(np.float16)
            zero = np.zeros((B, Hkv, C), np.float16)
            zero[:, :, :n_occ] = rng.uniform(-4.5, -1.5, size=(B, Hkv, n_occ)).astype(np.float16)
            out[name + "_codes"], out[name + "_scale"], out[name + "_zero"] = codes, scale, zero
        else:
            raise ValueError(fmt)
    scores = np.zeros((B, Hkv, C), np.float32)
    scores[:, :, :n_occ] = rng.uniform(0.0, prior_hi, size=(B, Hkv, n_occ)).astype(np.float32)
    token_pos = np.full((B, Hkv, C), -1, np.int32)
    token_pos[:, :, :n_occ] = np.arange(n_occ, dtype=np.int32)
    out["scores"], out["token_pos"] = scores, token_pos
    return out
