"""Helpers for the GPU parity tests: moving seeded inputs to the device,
tolerance checks taken from the stated bars, and the tie-band check of the
eviction set."""

from __future__ import annotations

import numpy as np
import torch

from h2o_kv_cache_sdpa_amd import workloads as W

DEV = "cuda:0"

# Tolerances (bars stated for the chunk step):
OUT_F32_ABS = 1e-5    # fp32 output: max abs error
OUT_BF16_REL = 2e-2   # bf16 output: per row, max|o - ref| <= 2e-2 * max|ref|
WSUM_REL = 1e-3       # summed weights and updated scores: elementwise relative
TIE_BAND = 1e-6       # slots within 1e-6 relative of the T-th smallest score may swap


def to_dev(stored):
    """workloads.Stored -> torch tensor on the GPU in the storage dtype."""
    if stored.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(stored.raw).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(stored.raw)).to(DEV)


def f64_to_dev(x64, dtype):
    return to_dev(W.to_storage(x64, dtype))


def out_to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def check_out(out, ref, dtype, what="out"):
    o = out_to_np(out)
    if dtype == "f32":
        err = np.abs(o - ref).max()
        assert err <= OUT_F32_ABS, f"{what}: max abs err {err:.3e}"
        return err
    num = np.abs(o - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    rel = num / np.maximum(den, 1e-30)
    assert rel.max() <= OUT_BF16_REL, f"{what}: worst row rel err {rel.max():.3e}"
    return rel.max()


def check_rel(got, ref, T, qg, what):
    got = np.asarray(got, np.float64)
    if got.size == 0:
        return 0.0
    bound = WSUM_REL * np.abs(ref) + 1e-20 * T * qg
    bad = np.abs(got - ref) > bound
    if bad.any():
        idx = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} elements out of tolerance, first at {tuple(idx)}: "
                             f"got {got[tuple(idx)]!r} ref {ref[tuple(idx)]!r}")
    return (np.abs(got - ref) / np.maximum(np.abs(ref), 1e-30)).max()


def check_selection(gpu_slots, oracle_slots, phi_upd, n_occ, C, T):
    """Replay-log parity.  Fill steps must match exactly.  Evicting steps: the
    GPU set G may differ from the oracle set R only among slots whose oracle
    score lies within TIE_BAND relative of the oracle's T-th smallest score;
    the log row must be G in ascending order.  Returns the number of groups
    whose set differed (inside the band)."""
    gpu_slots = np.asarray(gpu_slots)
    if n_occ + T <= C:
        assert (gpu_slots == oracle_slots).all(), "fill step: slot log differs"
        return 0
    differ = 0
    B, H = gpu_slots.shape[:2]
    idx = np.arange(C)
    for b in range(B):
        for g in range(H):
            row = gpu_slots[b, g]
            assert (np.diff(row) > 0).all(), f"({b},{g}) log not strictly ascending"
            assert row.min() >= 0 and row.max() < C
            phi = phi_upd[b, g]
            order = np.lexsort((idx, phi))
            theta = phi[order[T - 1]]
            G, R = set(row.tolist()), set(oracle_slots[b, g].tolist())
            sym = G ^ R
            if sym:
                band = np.abs(phi[list(sym)] - theta) <= TIE_BAND * abs(theta)
                assert band.all(), (f"({b},{g}) out-of-band swap: slots "
                                    f"{sorted(np.array(list(sym))[~band].tolist())[:8]} theta {theta!r}")
                differ += 1
    return differ
