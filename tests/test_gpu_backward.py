"""GPU parity of h2o_sdpa_backward (gradients of the chunk attention) against
the fp64 oracle: dq, the cache rows' dk/dv and the chunk's dk/dv, at sizes
spanning several key tiles and row blocks with ragged tails, an empty cache
(prefill square), a full cache and single-token chunks; determinism; rows of
the cache gradients past n_occ are left alone."""

import numpy as np
import pytest
import torch

from h2o_kv_cache_sdpa_amd import api
from h2o_kv_cache_sdpa_amd import workloads as W
from oracle import h2o_oracle as O
from tests.gpu_support import DEV, to_dev

pytestmark = pytest.mark.gpu

# Gradient bar (bf16 inputs; P and dS enter the products as bf16): per
# (batch, head) slice, max|g - g_ref| <= GRAD_REL * max|g_ref|, and over the
# whole tensor ||g - g_ref||_F <= GRAD_FRO * ||g_ref||_F.
GRAD_REL = 2e-2
GRAD_FRO = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    api.lib()


def _check_grad(g, ref, what):
    g = g.cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, what
    assert np.isfinite(g).all(), f"{what}: non-finite"
    flat_g = g.reshape(g.shape[0] * g.shape[1], -1)
    flat_r = ref.reshape(ref.shape[0] * ref.shape[1], -1)
    for s in range(flat_g.shape[0]):
        scale = np.abs(flat_r[s]).max()
        err = np.abs(flat_g[s] - flat_r[s]).max()
        assert err <= GRAD_REL * scale + 1e-12, f"{what} slice {s}: max err {err:.3e} vs max {scale:.3e}"
    fro = np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-30)
    assert fro <= GRAD_FRO, f"{what}: relative Frobenius error {fro:.3e}"


def _run(case, seed=70):
    B, Hq, Hkv, C, T, n_occ = case
    D = 128
    k, v, _, _, _ = W.random_cache([seed, B, Hq, C, T, n_occ], B, Hkv, C, D, n_occ, "bf16", hh_frac=0.05)
    ch = W.random_chunk([seed, 1, B, Hq, C, T], B, Hq, Hkv, T, D, "bf16", hh_frac=0.05)
    rng = np.random.default_rng([seed, 2, B, Hq, C, T])
    dout_st = W.to_storage(rng.standard_normal((B, Hq, T, D)), "bf16")
    dims = api.make_dims(B, Hq, Hkv, D, C, T)
    ws = torch.empty(api.workspace_bytes(dims), dtype=torch.uint8, device=DEV)
    kd, vd = to_dev(k), to_dev(v)
    bufs = api.cache_struct(kd, vd)
    q, kn, vn, dout = to_dev(ch["q"]), to_dev(ch["k"]), to_dev(ch["v"]), to_dev(dout_st)
    out = torch.empty_like(q)
    wsum = torch.empty(B, Hkv, n_occ + T, dtype=torch.float32, device=DEV)
    lse = torch.empty(B, Hq, T, dtype=torch.float32, device=DEV)
    api.h2o_sdpa_scoresum(dims, bufs, n_occ, q, kn, vn, out, wsum, lse, ws)
    sentinel = 7.25
    dq = torch.empty(B, Hq, T, D, dtype=torch.float32, device=DEV)
    dkc = torch.full((B, Hkv, C, D), sentinel, dtype=torch.float32, device=DEV)
    dvc = torch.full((B, Hkv, C, D), sentinel, dtype=torch.float32, device=DEV)
    dkn = torch.empty(B, Hkv, T, D, dtype=torch.float32, device=DEV)
    dvn = torch.empty(B, Hkv, T, D, dtype=torch.float32, device=DEV)
    api.h2o_sdpa_backward(dims, bufs, n_occ, q, kn, vn, lse, dout, dq, dkc, dvc, dkn, dvn, ws)
    torch.cuda.synchronize()
    scale = float(np.float32(1.0 / np.sqrt(D)))
    # the exact gradient of the chunk attention at the stored (bf16) inputs
    ref = O.attend_backward(ch["q"].f64, k.f64, v.f64, n_occ, ch["k"].f64, ch["v"].f64, scale, dout_st.f64)
    return (dq, dkc, dvc, dkn, dvn), ref, sentinel


BWD_CASES = [
    # B, Hq, Hkv, C, T, n_occ
    (1, 8, 2, 512, 64, 448),
    (1, 8, 2, 256, 256, 0),      # prefill: causal square on an empty cache
    (2, 8, 4, 1024, 128, 1024),  # full cache
    (1, 16, 2, 700, 50, 650),    # ragged key and row tails, q_g = 8
    (1, 32, 8, 4096, 1, 4096),   # one query per head
    (1, 4, 1, 300, 37, 0),
    (1, 8, 8, 192, 17, 100),     # q_g = 1
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "-".join(map(str, c)))
def test_backward_parity(case):
    print(f"backward case {case}", flush=True)
    B, Hq, Hkv, C, T, n_occ = case
    (dq, dkc, dvc, dkn, dvn), (rq, rkc, rvc, rkn, rvn), sentinel = _run(case)
    _check_grad(dq, rq, "dq")
    _check_grad(dkn, rkn, "dk_new")
    _check_grad(dvn, rvn, "dv_new")
    if n_occ:
        _check_grad(dkc[:, :, :n_occ], rkc, "dk_cache")
        _check_grad(dvc[:, :, :n_occ], rvc, "dv_cache")
    assert (dkc[:, :, n_occ:] == sentinel).all() and (dvc[:, :, n_occ:] == sentinel).all(), \
        "cache gradient rows past n_occ were written"


def test_backward_deterministic():
    case = (1, 8, 2, 1024, 200, 900)
    a, _, _ = _run(case, seed=71)
    b, _, _ = _run(case, seed=71)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_rejects_quantised_cache():
    dims = api.make_dims(1, 8, 2, 128, 256, 16, "bf16", "int8")
    ws = torch.empty(api.workspace_bytes(dims), dtype=torch.uint8, device=DEV)
    t = torch.zeros(1, 8, 16, 128, dtype=torch.bfloat16, device=DEV)
    t2 = torch.zeros(1, 2, 16, 128, dtype=torch.bfloat16, device=DEV)
    f = torch.zeros(1, 8, 16, 128, dtype=torch.float32, device=DEV)
    f2 = torch.zeros(1, 2, 16, 128, dtype=torch.float32, device=DEV)
    k = torch.zeros(1, 2, 256, 128, dtype=torch.int8, device=DEV)
    s = torch.zeros(1, 2, 256, dtype=torch.float16, device=DEV)
    bufs = api.cache_struct(k, k, k_scale=s, v_scale=s)
    lse = torch.zeros(1, 8, 16, dtype=torch.float32, device=DEV)
    with pytest.raises(api.H2OError) as e:
        api.h2o_sdpa_backward(dims, bufs, 0, t, t2, t2, lse, t, f, None, None, f2, f2, ws)
    assert e.value.status == api.H2O_EUNSUPPORTED
