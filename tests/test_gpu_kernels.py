"""GPU parity of each entry point against the fp64 oracle, element by element,
at sizes the oracle finishes in seconds (several tiles plus ragged tails) and
at the edge cases: empty cache, q_g = 1 and 8, D = 64, ties, signed zeros,
constant and tiny rows for the quantisers."""

import numpy as np
import pytest
import torch

from h2o_kv_cache_sdpa_amd import api
from h2o_kv_cache_sdpa_amd import workloads as W
from oracle import h2o_oracle as O
from tests.gpu_support import (DEV, check_out, check_rel, check_selection, f64_to_dev, out_to_np,
                               to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    api.lib()


def _cache_state(seed, fmt, dtype, B, Hkv, C, D, n_occ):
    """Device cache buffers plus the oracle's float64 view of them."""
    if fmt == "native":
        k, v, scores, tp, _ = W.random_cache(seed, B, Hkv, C, D, n_occ, dtype, hh_frac=0.05)
        dev = dict(k=to_dev(k), v=to_dev(v))
        k64, v64 = k.f64, v.f64
    else:
        arr = W.random_quant_cache(seed, B, Hkv, C, D, n_occ, fmt)
        scores, tp = arr["scores"], arr["token_pos"]
        dev = {}
        for name in ("k", "v"):
            dev[name] = torch.from_numpy(arr[name + "_codes"]).to(DEV)
            dev[name + "_scale"] = torch.from_numpy(arr[name + "_scale"]).to(DEV)
            if fmt == "int4":
                dev[name + "_zero"] = torch.from_numpy(arr[name + "_zero"]).to(DEV)
        if fmt == "int8":
            k64 = O.dequantize_int8(arr["k_codes"], arr["k_scale"])
            v64 = O.dequantize_int8(arr["v_codes"], arr["v_scale"])
        else:
            k64 = O.dequantize_int4(arr["k_codes"], arr["k_scale"], arr["k_zero"])
            v64 = O.dequantize_int4(arr["v_codes"], arr["v_scale"], arr["v_zero"])
    dev["scores"] = torch.from_numpy(scores).to(DEV)
    dev["token_pos"] = torch.from_numpy(tp).to(DEV)
    return dev, k64, v64, scores, tp


def _bufs(dev):
    return api.cache_struct(dev["k"], dev["v"], dev["scores"], dev["token_pos"], dev.get("k_scale"),
                            dev.get("v_scale"), dev.get("k_zero"), dev.get("v_zero"))


SDPA_CASES = [
    # dtype, fmt, B, Hq, Hkv, D, C, T, n_occ
    ("bf16", "native", 1, 8, 2, 128, 512, 100, 0),
    ("bf16", "native", 2, 8, 2, 128, 512, 100, 300),
    ("bf16", "native", 1, 4, 1, 64, 256, 64, 256),
    ("bf16", "native", 1, 8, 8, 128, 1000, 77, 1000),
    ("bf16", "native", 1, 16, 2, 128, 700, 50, 700),
    ("bf16", "native", 1, 8, 2, 64, 333, 129, 201),
    ("bf16", "native", 1, 8, 2, 128, 4096, 64, 4096),   # pass A split over 16 key ranges
    ("bf16", "native", 2, 8, 2, 128, 2048, 16, 2000),   # split, ragged occupancy
    ("bf16", "native", 1, 32, 8, 128, 8192, 1, 8192),   # one query per head (decode)
    ("bf16", "native", 1, 8, 2, 128, 700, 3, 0),        # tiny chunk, empty cache
    # at most 16 query rows per KV group: sums from pass A's stored logits
    ("bf16", "native", 1, 16, 4, 128, 5000, 4, 4321),   # 16 rows, ragged occupancy
    ("bf16", "int8", 2, 16, 4, 128, 3000, 4, 2990),
    ("bf16", "int8", 1, 32, 8, 128, 8192, 1, 8192),     # int8 decode
    ("bf16", "int4", 1, 8, 2, 128, 900, 2, 64),
    ("bf16", "native", 1, 4, 1, 128, 64, 1, 0),         # one key in all
    # capacities that are not a multiple of 4: each group's fp16 factor rows
    # start 2-byte aligned (the short pass loads a lane's four factors at once)
    ("bf16", "int8", 2, 16, 4, 128, 2051, 1, 2051),
    ("bf16", "int4", 1, 16, 4, 128, 1999, 4, 1998),
    ("bf16", "native", 1, 32, 8, 128, 3001, 2, 2999),
    # short chunks with other group sizes: q_g = 1, 2, 8 (16 rows each)
    ("bf16", "int4", 1, 8, 8, 128, 1000, 16, 1000),
    ("bf16", "int8", 1, 16, 8, 128, 777, 8, 700),
    ("bf16", "native", 1, 64, 8, 128, 1500, 2, 1500),
    # 8/4-bit short chunks with no full cache tile: an empty cache, and one
    # tile that mixes cached codes with the chunk's own keys
    ("bf16", "int8", 1, 8, 2, 128, 64, 1, 0),
    ("bf16", "int4", 1, 8, 2, 128, 100, 3, 37),
    # prefill: the first chunk fills an empty cache (a causal square)
    ("bf16", "native", 1, 8, 2, 128, 2048, 2048, 0),
    ("bf16", "int8", 1, 8, 2, 128, 1024, 1024, 0),
    ("bf16", "native", 2, 8, 4, 64, 640, 640, 0),
    ("bf16", "native", 1, 8, 2, 128, 1100, 1100, 0),   # pass B pairs key blocks (5: middle one alone)
    ("bf16", "int4", 1, 8, 2, 128, 768, 768, 0),       # 3 key blocks
    ("bf16", "int8", 1, 8, 2, 128, 4096, 16, 4096),     # quantised pass A split 16 ways
    ("bf16", "int4", 1, 32, 8, 128, 4096, 1, 4096),     # quantised decode, split
    ("bf16", "int4", 2, 8, 2, 128, 3000, 40, 2960),     # split, ragged
    ("bf16", "int8", 1, 8, 2, 128, 512, 100, 300),
    ("bf16", "int8", 1, 8, 2, 64, 300, 40, 300),
    ("bf16", "int4", 2, 8, 2, 128, 512, 96, 512),
    ("bf16", "int4", 1, 8, 2, 64, 300, 40, 200),
    # more than 512 pass-B blocks: chunk-only keys folded into the full key
    # blocks as 32-key slices (ragged last slice, ragged rows, q_g 1/2/4)
    ("bf16", "native", 2, 16, 16, 128, 4096, 300, 4000),
    ("bf16", "native", 1, 128, 32, 128, 4096, 200, 4040),
    ("bf16", "int8", 2, 32, 16, 128, 4096, 256, 4096),
    ("bf16", "int4", 2, 32, 16, 128, 4096, 200, 3900),
    ("f32", "native", 1, 4, 1, 64, 256, 32, 256),
    ("f32", "native", 1, 8, 2, 128, 300, 50, 123),
    ("f32", "native", 1, 8, 2, 128, 300, 50, 0),
    ("f32", "int8", 1, 8, 2, 64, 256, 32, 200),
    ("f32", "int4", 1, 8, 2, 128, 256, 32, 256),
]


@pytest.mark.parametrize("case", SDPA_CASES, ids=lambda c: "-".join(map(str, c)))
def test_sdpa_scoresum_parity(case):
    dtype, fmt, B, Hq, Hkv, D, C, T, n_occ = case
    print(f"sdpa case {case}", flush=True)
    seed = [31, B, Hq, Hkv, D, C, T, n_occ]
    dev, k64, v64, _, _ = _cache_state(seed, fmt, dtype, B, Hkv, C, D, n_occ)
    ch = W.random_chunk(seed + [1], B, Hq, Hkv, T, D, dtype, hh_frac=0.05)
    dims = api.make_dims(B, Hq, Hkv, D, C, T, dtype, fmt)
    ws = torch.empty(api.workspace_bytes(dims), dtype=torch.uint8, device=DEV)
    q, kn, vn = to_dev(ch["q"]), to_dev(ch["k"]), to_dev(ch["v"])
    out = torch.empty_like(q)
    wsum = torch.empty(B, Hkv, n_occ + T, dtype=torch.float32, device=DEV)
    lse = torch.empty(B, Hq, T, dtype=torch.float32, device=DEV)
    api.h2o_sdpa_scoresum(dims, _bufs(dev), n_occ, q, kn, vn, out, wsum, lse, ws)
    torch.cuda.synchronize()
    scale = float(np.float32(1 / np.sqrt(D)))
    ref_o, ref_w, ref_lse = O.attend_chunk(ch["q"].f64, k64, v64, n_occ, ch["k"].f64, ch["v"].f64, scale)
    check_out(out, ref_o, dtype)
    check_rel(wsum.cpu().numpy(), ref_w, T, Hq // Hkv, "wsum")
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=2e-6, atol=2e-5)


def test_sdpa_deterministic():
    B, Hq, Hkv, D, C, T, n_occ = 1, 8, 2, 128, 1024, 128, 1024
    dev, *_ = _cache_state([32], "native", "bf16", B, Hkv, C, D, n_occ)
    ch = W.random_chunk([33], B, Hq, Hkv, T, D, "bf16")
    dims = api.make_dims(B, Hq, Hkv, D, C, T)
    ws = torch.empty(api.workspace_bytes(dims), dtype=torch.uint8, device=DEV)
    q, kn, vn = to_dev(ch["q"]), to_dev(ch["k"]), to_dev(ch["v"])
    res = []
    for _ in range(2):
        out = torch.empty_like(q)
        wsum = torch.empty(B, Hkv, n_occ + T, dtype=torch.float32, device=DEV)
        api.h2o_sdpa_scoresum(dims, _bufs(dev), n_occ, q, kn, vn, out, wsum, None, ws)
        res.append((out.clone(), wsum.clone()))
    torch.cuda.synchronize()
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])


def test_sdpa_zero_queries_closed_form():
    """Q = 0: each row spreads its weight uniformly over the visible keys."""
    B, Hq, Hkv, D, C, T, n_occ = 1, 8, 2, 128, 640, 96, 640
    dev, k64, v64, _, _ = _cache_state([34], "native", "bf16", B, Hkv, C, D, n_occ)
    ch = W.random_chunk([35], B, Hq, Hkv, T, D, "bf16", q_zero=True)
    dims = api.make_dims(B, Hq, Hkv, D, C, T)
    ws = torch.empty(api.workspace_bytes(dims), dtype=torch.uint8, device=DEV)
    q, kn, vn = to_dev(ch["q"]), to_dev(ch["k"]), to_dev(ch["v"])
    out = torch.empty_like(q)
    wsum = torch.empty(B, Hkv, n_occ + T, dtype=torch.float32, device=DEV)
    api.h2o_sdpa_scoresum(dims, _bufs(dev), n_occ, q, kn, vn, out, wsum, None, ws)
    torch.cuda.synchronize()
    qg = Hq // Hkv
    harm = lambda n: sum(1.0 / k for k in range(1, n + 1))
    w = wsum.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(w[..., :n_occ], qg * (harm(n_occ + T) - harm(n_occ)), rtol=1e-5)
    expect_new = [qg * sum(1.0 / (n_occ + i + 1) for i in range(t, T)) for t in range(T)]
    np.testing.assert_allclose(w[..., n_occ:], np.broadcast_to(expect_new, w[..., n_occ:].shape), rtol=1e-5)
    # every old slot got the identical sum (same operation sequence per column)
    assert (w[..., :n_occ] == w[..., :1]).all()


# ---------------------------------------------------------------------------
# eviction
# ---------------------------------------------------------------------------

def _run_evict(scores, w, n_occ, T, pos=1000, token_pos=True, policy="h2o", two_pass=False):
    """two_pass: hand the call a workspace, which lets short chunks select over
    per-slice candidate lists (same result by construction)."""
    B, H, C = scores.shape
    dims = api.make_dims(B, 8 * H, H, 128, C, T, policy=policy)
    sc = torch.from_numpy(scores.copy()).to(DEV)
    tp = torch.from_numpy(np.arange(B * H * C, dtype=np.int32).reshape(B, H, C) % 977).to(DEV) if token_pos else None
    wd = torch.from_numpy(w).to(DEV)
    slots = torch.empty(B, H, T, dtype=torch.int32, device=DEV)
    k = torch.empty(16, dtype=torch.uint8, device=DEV)
    bufs = api.cache_struct(k, k, sc, tp)
    ws = torch.empty(api.workspace_bytes(dims), dtype=torch.uint8, device=DEV) if two_pass else None
    api.h2o_evict_topk(dims, bufs, n_occ, pos, wd, slots, ws)
    torch.cuda.synchronize()
    return sc.cpu().numpy(), (tp.cpu().numpy() if token_pos else None), slots.cpu().numpy()


EVICT_CASES = [
    # B, H, C, T, n_occ
    (1, 1, 256, 32, 256),
    (1, 8, 32768, 2048, 32768),
    (2, 3, 16384, 1024, 16384),
    (1, 2, 1000, 100, 1000),
    (1, 2, 512, 64, 128),      # filling
    (1, 2, 512, 64, 0),        # first chunk
    (1, 1, 65536, 64, 65536),  # largest supported cache
    (1, 1, 300, 300, 300),     # T == C
    (4, 8, 2048, 1, 2048),     # single-token chunk
    (1, 8, 32768, 1, 32768),   # decode on the 32K-slot cache
    (1, 8, 32768, 16, 32768),
    (2, 3, 16384, 128, 16384),
    (1, 2, 3082, 64, 3082),    # last 1024-slot slice shorter than the chunk
    # chunks of 2..8 tokens: rounds of the block minimum in both selection passes
    (1, 8, 32768, 4, 32768),
    (2, 3, 4096, 8, 4096),
    (1, 2, 3075, 5, 3075),     # last slice (3 slots) shorter than the chunk
]


@pytest.mark.parametrize("two_pass", [False, True], ids=["one_pass", "ws"])
@pytest.mark.parametrize("case", EVICT_CASES, ids=lambda c: "-".join(map(str, c)))
def test_evict_parity(case, two_pass):
    B, H, C, T, n_occ = case
    print(f"evict case {case} two_pass={two_pass}", flush=True)
    rng = np.random.default_rng([40, B, H, C, T])
    scores = np.zeros((B, H, C), np.float32)
    scores[..., :n_occ] = rng.uniform(0, 50, (B, H, n_occ)).astype(np.float32)
    w = rng.exponential(0.3, (B, H, n_occ + T)).astype(np.float32)
    pos = 5000
    sc, tp, slots = _run_evict(scores, w, n_occ, T, pos, two_pass=two_pass)
    phi_upd = O.update_scores(scores.astype(np.float64), w.astype(np.float64), n_occ, C, T)
    ref = O.bottom_t(phi_upd, n_occ, C, T)
    check_selection(slots, ref, phi_upd, n_occ, C, T)
    # stored scores: fp32 sum for kept occupied slots, own sums for the new ones
    expect = scores.copy()
    expect[..., :n_occ] = scores[..., :n_occ] + w[..., :n_occ]  # float32 addition
    tp0 = np.arange(B * H * C, dtype=np.int32).reshape(B, H, C) % 977
    for b in range(B):
        for g in range(H):
            expect[b, g, slots[b, g]] = w[b, g, n_occ:]
            tp0[b, g, slots[b, g]] = pos + np.arange(T)
    np.testing.assert_array_equal(sc, expect)
    np.testing.assert_array_equal(tp, tp0)
    # and the kept scores agree with the oracle's fp64 accumulation
    kept = np.ones((B, H, C), bool)
    for b in range(B):
        for g in range(H):
            kept[b, g, slots[b, g]] = False
    kept[..., n_occ:] = False
    check_rel(sc[kept], phi_upd[kept], T, 1, "scores")


POLICY_CASES = [
    # B, H, C, T, n_occ
    (1, 2, 1000, 100, 1000),
    (4, 8, 32768, 1024, 32768),  # the int4 batch workload's shape
    (3, 2, 4096, 512, 4096),
    (2, 2, 512, 64, 128),        # filling: the same under every policy
    (2, 1, 300, 300, 300),       # T == C
    (2, 2, 8192, 16, 8192),      # short chunk
    (2, 2, 8192, 4, 8192),       # 2..8 tokens: rounds of the block minimum
]


@pytest.mark.parametrize("two_pass", [False, True], ids=["one_pass", "ws"])
@pytest.mark.parametrize("policy", ["h2o_norm", "h2o_orig"])
@pytest.mark.parametrize("case", POLICY_CASES, ids=lambda c: "-".join(map(str, c)))
def test_evict_policy_parity(case, policy, two_pass):
    B, H, C, T, n_occ = case
    print(f"evict {policy} case {case} two_pass={two_pass}", flush=True)
    rng = np.random.default_rng([42, B, H, C, T])
    scores = np.zeros((B, H, C), np.float32)
    scores[..., :n_occ] = rng.uniform(0, 50, (B, H, n_occ)).astype(np.float32)
    w = rng.exponential(0.3, (B, H, n_occ + T)).astype(np.float32)
    pos = 5000
    tp0 = np.arange(B * H * C, dtype=np.int32).reshape(B, H, C) % 977
    sc, tp, slots = _run_evict(scores, w, n_occ, T, pos, policy=policy, two_pass=two_pass)
    phi_upd = O.update_scores(scores.astype(np.float64), w.astype(np.float64), n_occ, C, T)
    key = O.selection_key(phi_upd, tp0, pos, T, policy) if n_occ == C else phi_upd
    ref = O.bottom_t(key, n_occ, C, T)
    check_selection(slots, ref, key, n_occ, C, T)
    if policy == "h2o_orig":
        assert (slots == slots[:1]).all(), "batch rows selected different slots"
    expect = scores.copy()
    expect[..., :n_occ] = scores[..., :n_occ] + w[..., :n_occ]
    tp_exp = tp0.copy()
    for b in range(B):
        for g in range(H):
            expect[b, g, slots[b, g]] = w[b, g, n_occ:]
            tp_exp[b, g, slots[b, g]] = pos + np.arange(T)
    np.testing.assert_array_equal(sc, expect)
    np.testing.assert_array_equal(tp, tp_exp)


@pytest.mark.parametrize("two_pass", [False, True], ids=["one_pass", "ws"])
@pytest.mark.parametrize("T", [512, 16, 8, 4, 1])
def test_evict_ties_resolve_to_lower_index(T, two_pass):
    rng = np.random.default_rng(41)
    B, H, C = 2, 4, 4096
    scores = (rng.integers(0, 9, (B, H, C)) * 0.25).astype(np.float32)  # many exact ties
    w = np.zeros((B, H, C + T), np.float32)
    _, _, slots = _run_evict(scores, w, C, T, two_pass=two_pass)
    ref = O.bottom_t(scores.astype(np.float64), C, C, T)
    np.testing.assert_array_equal(slots, ref)
    scores[:] = 3.0  # all tied: lowest indices
    _, _, slots = _run_evict(scores, w, C, T, token_pos=False, two_pass=two_pass)
    assert (slots == np.arange(T)).all()
    # ties that straddle slices: the tied minimum sits in the last slices only
    scores[:] = 3.0
    scores[..., 3000:] = 1.0
    _, _, slots = _run_evict(scores, w, C, T, token_pos=False, two_pass=two_pass)
    assert (slots == 3000 + np.arange(T)).all()


def test_evict_signed_zero_and_negative_scores():
    B, H, C, T = 1, 1, 64, 8
    scores = np.full((B, H, C), 5.0, np.float32)
    scores[0, 0, [3, 9, 20]] = [-0.0, 0.0, -0.0]
    scores[0, 0, [40, 41]] = [-1.5, -2.0]
    scores[0, 0, [50, 60]] = [1e-30, -1e-30]
    w = np.zeros((B, H, C + T), np.float32)
    _, _, slots = _run_evict(scores, w, C, T)
    ref = O.bottom_t(scores.astype(np.float64), C, C, T)
    np.testing.assert_array_equal(slots, ref)


# ---------------------------------------------------------------------------
# slot overwrite and quantisation
# ---------------------------------------------------------------------------

def _special_rows(x):
    x = x.copy()
    x[0, 0, 0] = 0.0                  # all-zero row
    x[0, 0, 1] = 1.25                 # constant row
    x[0, 0, 2] = 0.0
    x[0, 0, 2, 5] = -300.0            # one large element
    x[0, 0, 3] *= 1e-6                # tiny values (fp16 subnormal scales)
    x[0, 0, 4] *= 1e-9                # scale rounds to zero in fp16
    return x


def _bits(a):
    """Raw bytes of an array, for bit-exact comparison."""
    return np.ascontiguousarray(a).view(np.uint8)


@pytest.mark.parametrize("fmt,dtype,D", [("native", "bf16", 128), ("native", "f32", 64),
                                         ("native", "bf16", 64), ("int8", "bf16", 128),
                                         ("int8", "f32", 64), ("int4", "bf16", 128),
                                         ("int4", "f32", 128), ("int4", "bf16", 64)])
def test_kv_write_parity(fmt, dtype, D):
    B, Hkv, C, T = 2, 3, 300, 40
    rng = np.random.default_rng([42, D])
    kn = W.to_storage(_special_rows(rng.standard_normal((B, Hkv, T, D)) * 2), dtype)
    vn = W.to_storage(_special_rows(rng.standard_normal((B, Hkv, T, D))), dtype)
    slots = np.stack([np.stack([np.sort(rng.choice(C, T, replace=False)) for _ in range(Hkv)])
                      for _ in range(B)]).astype(np.int32)
    dims = api.make_dims(B, 8 * Hkv, Hkv, D, C, T, dtype, fmt)
    dev = {}
    if fmt == "native":
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        dev["k"] = torch.randn(B, Hkv, C, D, device=DEV).to(tdt)
        dev["v"] = torch.randn(B, Hkv, C, D, device=DEV).to(tdt)
    else:
        shape = (B, Hkv, C, D) if fmt == "int8" else (B, Hkv, C, D // 2)
        cdt = torch.int8 if fmt == "int8" else torch.uint8
        for n in ("k", "v"):
            dev[n] = torch.randint(0, 100, shape, device=DEV).to(cdt)
            dev[n + "_scale"] = torch.rand(B, Hkv, C, device=DEV).half()
            if fmt == "int4":
                dev[n + "_zero"] = torch.rand(B, Hkv, C, device=DEV).half()
    before = {n: t.view(torch.uint8).cpu().numpy().copy() if t.dtype == torch.bfloat16 else t.cpu().numpy().copy()
              for n, t in dev.items()}
    bufs = api.cache_struct(dev["k"], dev["v"], None, None, dev.get("k_scale"), dev.get("v_scale"),
                            dev.get("k_zero"), dev.get("v_zero"))
    sl = torch.from_numpy(slots).to(DEV)
    if fmt == "native":
        api.kv_scatter(dims, bufs, to_dev(kn), to_dev(vn), sl)
    else:
        api.kv_quant_pack(dims, bufs, to_dev(kn), to_dev(vn), sl)
    torch.cuda.synchronize()
    after = {n: t.view(torch.uint8).cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()
             for n, t in dev.items()}
    values = {n: dev[n].float().cpu().numpy().astype(np.float64) for n in ("k", "v")}
    written = np.zeros((B, Hkv, C), bool)
    for b in range(B):
        for g in range(Hkv):
            written[b, g, slots[b, g]] = True
    for n, src in (("k", kn), ("v", vn)):
        for b in range(B):
            for g in range(Hkv):
                r = slots[b, g]
                if fmt == "native":
                    # rows are copied unchanged
                    np.testing.assert_array_equal(values[n][b, g, r], src.f64[b, g])
                elif fmt == "int8":
                    c, s_ = O.quantize_int8(src.f32[b, g])
                    np.testing.assert_array_equal(_bits(after[n][b, g, r]), _bits(c), err_msg=f"{n} codes")
                    np.testing.assert_array_equal(_bits(after[n + "_scale"][b, g, r]), _bits(s_))
                else:
                    c, s_, z = O.quantize_int4(src.f32[b, g])
                    np.testing.assert_array_equal(_bits(after[n][b, g, r]), _bits(c), err_msg=f"{n} codes")
                    np.testing.assert_array_equal(_bits(after[n + "_scale"][b, g, r]), _bits(s_))
                    np.testing.assert_array_equal(_bits(after[n + "_zero"][b, g, r]), _bits(z))
    # untouched slots keep their content
    for key in before:
        np.testing.assert_array_equal(_bits(after[key][~written]), _bits(before[key][~written]), err_msg=key)
    # the dequantising inspection helper returns the oracle's dequantised rows
    kout = torch.empty(B, Hkv, C, D, device=DEV)
    vout = torch.empty_like(kout)
    api.kv_dequant_unpack(dims, bufs, C, kout, vout)
    torch.cuda.synchronize()
    for n, outt in (("k", kout), ("v", vout)):
        if fmt == "int8":
            ref = O.dequantize_int8(after[n], after[n + "_scale"])
        elif fmt == "int4":
            ref = O.dequantize_int4(after[n], after[n + "_scale"], after[n + "_zero"])
        else:
            ref = values[n]
        np.testing.assert_array_equal(outt.cpu().numpy(), ref.astype(np.float32))
