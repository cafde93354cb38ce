"""Chunk-step streams through h2o_chunk_step against the fp64 oracle, step by
step, for the five workloads: tiny fp32 stream and the single bf16 step at full
size; the long bf16 / int8 / int4 streams with their structure (fill then
evict, heavy hitters, B) at reduced cache and chunk sizes; and consecutive
evicting steps of each long stream at full size with every KV group
recomputed by the oracle.

When the GPU picks a different slot than the oracle inside the tie band, the
GPU cache is reloaded from the oracle's state (inputs flow oracle -> GPU only)
so both continue from the same state; such steps are counted and reported."""

import numpy as np
import pytest
import torch

from h2o_kv_cache_sdpa_amd import workloads as W
from h2o_kv_cache_sdpa_amd.cache import H2OCache
from oracle import h2o_oracle as O
from tests.gpu_support import DEV, check_out, check_rel, check_selection, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _dev_bf16(x64):
    return to_dev(W.to_storage(x64, "bf16"))


def _load_gpu_from_oracle(gc: H2OCache, oc: O.OracleCache):
    """Copy the oracle's state into the GPU cache buffers (oracle -> GPU)."""
    if oc.fmt == "native":
        gc.k.copy_(to_dev(W.to_storage(oc.k, gc.dtype)))
        gc.v.copy_(to_dev(W.to_storage(oc.v, gc.dtype)))
    else:
        gc.k.copy_(torch.from_numpy(oc.k_codes).to(DEV))
        gc.v.copy_(torch.from_numpy(oc.v_codes).to(DEV))
        gc.k_scale.copy_(torch.from_numpy(oc.k_scale).to(DEV))
        gc.v_scale.copy_(torch.from_numpy(oc.v_scale).to(DEV))
        if oc.fmt == "int4":
            gc.k_zero.copy_(torch.from_numpy(oc.k_zero).to(DEV))
            gc.v_zero.copy_(torch.from_numpy(oc.v_zero).to(DEV))
    gc.scores.copy_(torch.from_numpy(oc.phi.astype(np.float32)).to(DEV))
    gc.token_pos.copy_(torch.from_numpy(oc.token_pos.astype(np.int32)).to(DEV))
    gc.n_occ, gc.pos = oc.n_occ, oc.pos


def _check_state(gc: H2OCache, oc: O.OracleCache, T, qg):
    n = oc.n_occ
    if oc.fmt == "native":
        for name in ("k", "v"):
            got = getattr(gc, name).float().cpu().numpy()[:, :, :n]
            np.testing.assert_array_equal(got, getattr(oc, name)[:, :, :n], err_msg=name)
    else:
        for name in ("k", "v"):
            np.testing.assert_array_equal(getattr(gc, name).cpu().numpy()[:, :, :n],
                                          getattr(oc, name + "_codes")[:, :, :n])
            np.testing.assert_array_equal(getattr(gc, name + "_scale").cpu().numpy()[:, :, :n].view(np.uint16),
                                          getattr(oc, name + "_scale")[:, :, :n].view(np.uint16))
            if oc.fmt == "int4":
                np.testing.assert_array_equal(getattr(gc, name + "_zero").cpu().numpy()[:, :, :n].view(np.uint16),
                                              getattr(oc, name + "_zero")[:, :, :n].view(np.uint16))
    np.testing.assert_array_equal(gc.token_pos.cpu().numpy()[:, :, :n], oc.token_pos[:, :, :n])
    check_rel(gc.scores.cpu().numpy()[:, :, :n], oc.phi[:, :, :n], T, qg, "scores")


def _run_stream(w: W.Workload, steps=None, policy="h2o"):
    gc = H2OCache(w.B, w.Hq, w.Hkv, w.D, w.C, w.T, dtype=w.dtype, cache_fmt=w.cache_fmt, device=DEV,
                  policy=policy)
    oc = O.OracleCache(w.B, w.Hq, w.Hkv, w.D, w.C, fmt=w.cache_fmt, policy=policy)
    if w.start_full:
        k, v, scores, tp, n = W.prefilled_cache(w)
        oc.k[:], oc.v[:] = k.f64, v.f64
        oc.phi[:] = scores.astype(np.float64)
        oc.token_pos[:] = tp
        oc.n_occ = oc.pos = n
        _load_gpu_from_oracle(gc, oc)
    resync = 0
    n_steps = w.steps if steps is None else steps
    for step in range(n_steps):
        ch = W.chunk(w, step)
        n_occ = oc.n_occ
        out, wsum, slots = gc.step(to_dev(ch["q"]), to_dev(ch["k"]), to_dev(ch["v"]))
        ref = oc.step(ch["q"].f64, ch["k"].f64, ch["v"].f64)
        torch.cuda.synchronize()
        err = check_out(out, ref["out"], w.dtype, f"step {step} out")
        werr = check_rel(wsum.cpu().numpy(), ref["w"], w.T, w.qg, f"step {step} wsum")
        differ = check_selection(slots.cpu().numpy(), ref["slots"], ref["rank_key"], n_occ, w.C, w.T)
        print(f"{w.name} step {step} n_occ {n_occ}: out err {err:.2e} wsum rel {werr:.2e} "
              f"in-band differ {differ}", flush=True)
        if differ:
            resync += 1
            _load_gpu_from_oracle(gc, oc)
        else:
            _check_state(gc, oc, w.T, w.qg)
    return resync


def test_stream_cfg1_tiny_f32_full():
    assert _run_stream(W.WORKLOADS[1]) == 0


def test_stream_cfg2_single_step_full():
    _run_stream(W.WORKLOADS[2])


def test_stream_cfg3_bf16_reduced():
    _run_stream(W.WORKLOADS[3].scaled(C=1024, T=64, n_fill=16, n_evict=12))


def test_stream_cfg4_int8_reduced():
    _run_stream(W.WORKLOADS[4].scaled(C=1024, T=64, n_fill=16, n_evict=12))


def test_stream_cfg5_int4_reduced():
    _run_stream(W.WORKLOADS[5].scaled(C=1024, T=32, n_fill=32, n_evict=10))


@pytest.mark.parametrize("policy", ["h2o_norm", "h2o_orig"])
def test_stream_policies_bf16_batch(policy):
    """The long bf16 stream's structure with B = 2 under the other two
    ranking policies ([LF] §3.1.1)."""
    _run_stream(W.WORKLOADS[3].scaled(B=2, C=1024, T=64, n_fill=16, n_evict=10), policy=policy)


@pytest.mark.parametrize("policy", ["h2o_norm", "h2o_orig"])
def test_stream_policies_short_chunks_batch(policy):
    """Four-token chunks, B = 2: the rounds selection, and the pick writing
    the K/V rows of every batch row it serves (one selection per KV head
    under h2o_orig)."""
    _run_stream(W.WORKLOADS[3].scaled(B=2, C=256, T=4, n_fill=64, n_evict=6), policy=policy)


@pytest.mark.parametrize("fmt,T,policy", [("int8", 1, "h2o"), ("int4", 1, "h2o_orig"), ("int8", 1, "h2o_norm"),
                                           ("int8", 4, "h2o_orig"), ("int4", 4, "h2o")])
def test_stream_short_chunks_quant(fmt, T, policy):
    """One- and four-token chunks into 8/4-bit caches, B = 2: the pick
    kernel quantises the chunk's K/V rows into the slots it took (for every
    batch row under h2o_orig); codes, scales and zero points bit for bit."""
    base = W.WORKLOADS[4] if fmt == "int8" else W.WORKLOADS[5]
    C = 128 if T == 1 else 256
    _run_stream(base.scaled(B=2, C=C, T=T, n_fill=C // T, n_evict=8, cache_fmt=fmt), policy=policy)


@pytest.mark.parametrize("T,policy", [(1, "h2o"), (4, "h2o"), (4, "h2o_orig"), (1, "h2o_norm")])
def test_stream_short_chunks_split_merge(T, policy):
    """Evicting one- and four-token steps on a prefilled 2048-slot cache, B = 2:
    pass A splits the keys (8 splits), and the selection's two slices each
    merge several output rows of every group from the split partials while
    summing the stored logits (both batch rows of a head under h2o_orig)."""
    w = W.WORKLOADS[2].scaled(B=2, C=2048, T=T, n_fill=0, n_evict=4, name=f"split_merge_t{T}")
    _run_stream(w, policy=policy)


@pytest.mark.parametrize("policy", ["h2o_norm", "h2o_orig"])
def test_stream_policies_int4_batch(policy):
    _run_stream(W.WORKLOADS[5].scaled(C=512, T=32, n_fill=16, n_evict=8), policy=policy)


def _replay_stream(w: W.Workload, steps):
    """Record the oracle's replay log on a stream, then replay it on the GPU
    (h2o_replay_step) beside the oracle's replay: outputs to tolerance, cache
    contents and positions bit for bit, scores untouched."""
    rec = O.OracleCache(w.B, w.Hq, w.Hkv, w.D, w.C, fmt=w.cache_fmt)
    oc = O.OracleCache(w.B, w.Hq, w.Hkv, w.D, w.C, fmt=w.cache_fmt)
    gc = H2OCache(w.B, w.Hq, w.Hkv, w.D, w.C, w.T, dtype=w.dtype, cache_fmt=w.cache_fmt, device=DEV)
    gc.scores.fill_(7.0)
    for step in range(steps):
        ch = W.chunk(w, step)
        q, kn, vn = ch["q"].f64, ch["k"].f64, ch["v"].f64
        log = rec.step(q, kn, vn)["slots"]
        ref = oc.replay_step(q, kn, vn, log)
        out = gc.replay_step(to_dev(ch["q"]), to_dev(ch["k"]), to_dev(ch["v"]),
                             torch.from_numpy(log.astype(np.int32)).to(DEV))
        torch.cuda.synchronize()
        err = check_out(out, ref, w.dtype, f"replay step {step} out")
        print(f"{w.name} replay step {step}: out err {err:.2e}", flush=True)
        oc.phi[:] = 7.0  # the replay keeps no scores; compare the rest of the state
        _check_state(gc, oc, w.T, w.qg)
    assert (gc.scores == 7.0).all()


@pytest.mark.parametrize("cfg", [1, 3, 4, 5])
def test_replay_stream(cfg):
    sizes = {1: {}, 3: dict(C=512, T=64), 4: dict(C=512, T=64), 5: dict(C=256, T=32)}[cfg]
    w = W.WORKLOADS[cfg].scaled(**sizes)
    _replay_stream(w, steps=min(w.steps, (w.C // w.T) + 6))


# ---------------------------------------------------------------------------
# full-size evicting steps, every KV group recomputed by the oracle
# ---------------------------------------------------------------------------

def _prefilled_pair(w: W.Workload):
    """A GPU cache and an oracle cache holding the same full cache of the
    workload's size (seed [cfg, 777]: random contents, 2 % heavy-hitter keys
    for bf16 caches, prior scores ~ U(0, 50), token_pos[j] = j)."""
    B, Hq, Hkv, D, C, T = w.B, w.Hq, w.Hkv, w.D, w.C, w.T
    gc = H2OCache(B, Hq, Hkv, D, C, T, dtype=w.dtype, cache_fmt=w.cache_fmt, device=DEV)
    oc = O.OracleCache(B, Hq, Hkv, D, C, fmt=w.cache_fmt)
    seed = [w.cfg_id, 777]
    if w.cache_fmt == "native":
        k, v, scores, tp, _ = W.random_cache(seed, B, Hkv, C, D, C, w.dtype, hh_frac=0.02)
        oc.k[:], oc.v[:] = k.f64, v.f64
    else:
        arr = W.random_quant_cache(seed, B, Hkv, C, D, C, w.cache_fmt)
        scores, tp = arr["scores"], arr["token_pos"]
        for name in ("k", "v"):
            getattr(oc, name + "_codes")[:] = arr[name + "_codes"]
            getattr(oc, name + "_scale")[:] = arr[name + "_scale"]
            if w.cache_fmt == "int4":
                getattr(oc, name + "_zero")[:] = arr[name + "_zero"]
        if w.cache_fmt == "int8":
            oc.k[:] = O.dequantize_int8(arr["k_codes"], arr["k_scale"])
            oc.v[:] = O.dequantize_int8(arr["v_codes"], arr["v_scale"])
        else:
            oc.k[:] = O.dequantize_int4(arr["k_codes"], arr["k_scale"], arr["k_zero"])
            oc.v[:] = O.dequantize_int4(arr["v_codes"], arr["v_scale"], arr["v_zero"])
    oc.phi[:] = scores.astype(np.float64)
    oc.token_pos[:] = tp
    oc.n_occ = oc.pos = C
    _load_gpu_from_oracle(gc, oc)
    return gc, oc


def _near_threshold(phi_gpu, phi_ref, T, window=1e-3):
    """Per KV group, the oracle's T-th smallest updated score theta; over the
    slots whose oracle score lies within `window` relative of theta, the
    largest |phi_gpu - phi_ref| / theta, and the number of slots inside the
    1e-6 tie band."""
    worst, in_band = 0.0, 0
    B, H, C = phi_ref.shape
    for b in range(B):
        for g in range(H):
            ref = phi_ref[b, g]
            theta = np.partition(ref, T - 1)[T - 1]
            near = np.abs(ref - theta) <= window * abs(theta)
            worst = max(worst, float((np.abs(phi_gpu[b, g][near] - ref[near]) / abs(theta)).max()))
            in_band += int((np.abs(ref - theta) <= 1e-6 * abs(theta)).sum())
    return worst, in_band


def _full_stream(w: W.Workload, n_steps):
    """Consecutive evicting steps on a full cache of the workload's size,
    starting at the stream's first evicting chunk.  Every step: the output,
    the summed weights and the selection of every (b, g) group against the
    oracle, then the cache state (contents bit for bit, positions, scores).
    Reports in-band swaps and the worst GPU score error near the threshold."""
    gc, oc = _prefilled_pair(w)
    C, T, qg = w.C, w.T, w.qg
    swaps = resync = 0
    for s in range(n_steps):
        ch = W.chunk(w, w.n_fill + s)
        phi_before = gc.scores.cpu().numpy()
        print(f"{w.name} full-size step {s}: GPU", flush=True)
        out, wsum, slots = gc.step(to_dev(ch["q"]), to_dev(ch["k"]), to_dev(ch["v"]))
        torch.cuda.synchronize()
        print(f"{w.name} full-size step {s}: oracle, {w.B * w.Hkv} groups", flush=True)
        ref = oc.step(ch["q"].f64, ch["k"].f64, ch["v"].f64)
        err = check_out(out, ref["out"], w.dtype, f"step {s} out")
        wsum_np = wsum.cpu().numpy()
        werr = check_rel(wsum_np, ref["w"], T, qg, f"step {s} wsum")
        differ = check_selection(slots.cpu().numpy(), ref["slots"], ref["rank_key"], C, C, T)
        # the selection kernel adds the sums to the scores in fp32
        phi_gpu = (phi_before + wsum_np[:, :, :C]).astype(np.float32).astype(np.float64)
        near_err, in_band = _near_threshold(phi_gpu, ref["phi_updated"], T)
        swaps += differ
        print(f"{w.name} full-size step {s}: out err {err:.2e} wsum rel {werr:.2e} "
              f"groups with in-band swaps {differ} slots in the tie band {in_band} "
              f"worst near-threshold score error / theta {near_err:.2e}", flush=True)
        assert near_err < 5e-7, "score error near the threshold reaches the tie band"
        if differ:
            resync += 1
            _load_gpu_from_oracle(gc, oc)
        else:
            _check_state(gc, oc, T, qg)
    print(f"{w.name}: {n_steps} full-size evicting steps, in-band swaps {swaps}, resyncs {resync}", flush=True)


@pytest.mark.timeout(900)
def test_full_stream_cfg3():
    _full_stream(W.WORKLOADS[3], 3)


@pytest.mark.timeout(900)
def test_full_stream_cfg4():
    _full_stream(W.WORKLOADS[4], 3)


@pytest.mark.timeout(900)
def test_full_stream_cfg5():
    _full_stream(W.WORKLOADS[5], 2)


def _full_step(w: W.Workload, groups_checked):
    """Prefilled full cache of the workload's size; one evicting step; the
    oracle recomputes the listed (b, g) groups completely."""
    B, Hq, Hkv, D, C, T = w.B, w.Hq, w.Hkv, w.D, w.C, w.T
    qg = w.qg
    gc = H2OCache(B, Hq, Hkv, D, C, T, dtype=w.dtype, cache_fmt=w.cache_fmt, device=DEV)
    seed = [w.cfg_id, 777]
    if w.cache_fmt == "native":
        k, v, scores, tp, _ = W.random_cache(seed, B, Hkv, C, D, C, w.dtype, hh_frac=0.02)
        gc.k.copy_(to_dev(k))
        gc.v.copy_(to_dev(v))
        k64, v64 = k.f64, v.f64
    else:
        arr = W.random_quant_cache(seed, B, Hkv, C, D, C, w.cache_fmt)
        scores, tp = arr["scores"], arr["token_pos"]
        for name in ("k", "v"):
            getattr(gc, name).copy_(torch.from_numpy(arr[name + "_codes"]).to(DEV))
            getattr(gc, name + "_scale").copy_(torch.from_numpy(arr[name + "_scale"]).to(DEV))
            if w.cache_fmt == "int4":
                getattr(gc, name + "_zero").copy_(torch.from_numpy(arr[name + "_zero"]).to(DEV))
        if w.cache_fmt == "int8":
            k64 = O.dequantize_int8(arr["k_codes"], arr["k_scale"])
            v64 = O.dequantize_int8(arr["v_codes"], arr["v_scale"])
        else:
            k64 = O.dequantize_int4(arr["k_codes"], arr["k_scale"], arr["k_zero"])
            v64 = O.dequantize_int4(arr["v_codes"], arr["v_scale"], arr["v_zero"])
    gc.scores.copy_(torch.from_numpy(scores).to(DEV))
    gc.token_pos.copy_(torch.from_numpy(tp).to(DEV))
    gc.n_occ, gc.pos = C, C
    ch = W.chunk(w, w.n_fill)  # the first evicting chunk of the stream
    out, wsum, slots = gc.step(to_dev(ch["q"]), to_dev(ch["k"]), to_dev(ch["v"]))
    torch.cuda.synchronize()
    wsum_np = wsum.cpu().numpy()
    # every query's weights sum to one: T*q_g per group, for all groups
    np.testing.assert_allclose(wsum_np.astype(np.float64).sum(-1), T * qg, rtol=1e-4)
    slots_np = slots.cpu().numpy()
    for (b, g) in groups_checked:
        print(f"{w.name}: oracle on group ({b},{g})", flush=True)
        sl = slice(g * qg, (g + 1) * qg)
        ref_o, ref_w, _ = O.attend_chunk(ch["q"].f64[b:b + 1, sl], k64[b:b + 1, g:g + 1],
                                         v64[b:b + 1, g:g + 1], C, ch["k"].f64[b:b + 1, g:g + 1],
                                         ch["v"].f64[b:b + 1, g:g + 1], float(np.float32(1 / np.sqrt(D))))
        check_out(out[b:b + 1, sl], ref_o, w.dtype, f"group ({b},{g}) out")
        check_rel(wsum_np[b:b + 1, g:g + 1], ref_w, T, qg, f"group ({b},{g}) wsum")
        phi_upd = O.update_scores(scores[b:b + 1, g:g + 1].astype(np.float64), ref_w, C, C, T)
        ref_slots = O.bottom_t(phi_upd, C, C, T)
        differ = check_selection(slots_np[b:b + 1, g:g + 1], ref_slots, phi_upd, C, C, T)
        print(f"group ({b},{g}) in-band differ {differ}", flush=True)


# short chunks on the full 32K-slot cache, in the launch configuration the
# small-T sweep times (key-split short-chunk pass A, stored logits with the
# folded combine, two-pass slot selection): every KV group recomputed

@pytest.mark.parametrize("fmt,T", [("native", 1), ("native", 4), ("native", 16), ("int8", 1), ("int4", 4)])
def test_full_step_short_chunks(fmt, T):
    w = W.WORKLOADS[3].scaled(T=T, cache_fmt=fmt, name=f"short_{fmt}_32k_t{T}")
    _full_step(w, [(0, g) for g in range(w.Hkv)])


def test_prefill_square_8k():
    """First chunk on an empty cache: n_occ = 0, T = C = 8192 (a causal square
    with summed weights); one KV group recomputed completely, the fill log and
    the per-group invariant sum(w) = T*q_g everywhere."""
    w = W.WORKLOADS[3].scaled(C=8192, T=8192, name="prefill_8k")
    B, Hq, Hkv, D, C, T = w.B, w.Hq, w.Hkv, w.D, w.C, w.T
    qg = w.qg
    gc = H2OCache(B, Hq, Hkv, D, C, T, dtype="bf16", cache_fmt="native", device=DEV)
    ch = W.chunk(w, 0)
    out, wsum, slots = gc.step(to_dev(ch["q"]), to_dev(ch["k"]), to_dev(ch["v"]))
    torch.cuda.synchronize()
    wsum_np = wsum.cpu().numpy()
    np.testing.assert_allclose(wsum_np.astype(np.float64).sum(-1), T * qg, rtol=1e-4)
    assert (slots.cpu().numpy() == np.arange(T)).all(), "fill log"
    g = 3
    sl = slice(g * qg, (g + 1) * qg)
    empty = np.zeros((1, 1, 0, D))
    ref_o, ref_w, _ = O.attend_chunk(ch["q"].f64[:, sl], empty, empty, 0, ch["k"].f64[:, g:g + 1],
                                     ch["v"].f64[:, g:g + 1], float(np.float32(1 / np.sqrt(D))))
    check_out(out[:, sl], ref_o, "bf16", "prefill out")
    check_rel(wsum_np[:, g:g + 1], ref_w, T, qg, "prefill wsum")
    # the cache now holds the chunk and its own sums
    np.testing.assert_array_equal(gc.k[:, g].cpu().view(torch.int16).numpy(),
                                  np.ascontiguousarray(ch["k"].raw[:, g]).view(np.int16))
    np.testing.assert_array_equal(gc.scores[:, g].cpu().numpy(), wsum_np[:, g])
