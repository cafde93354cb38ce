"""h2o_chunk_step_noalloc (workspace in the library's per-GPU device array)
against h2o_chunk_step (caller workspace): two calls in a row on the same
GPU, the second with a smaller problem, each compared with the existing
entry point on an identical cache: outputs, summed weights, replay log and
the cache state after the step."""

import numpy as np
import pytest
import torch

from h2o_kv_cache_sdpa_amd import api
from h2o_kv_cache_sdpa_amd import workloads as W
from h2o_kv_cache_sdpa_amd.cache import H2OCache
from tests.gpu_support import DEV, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    api.lib()


def _pair(w, seed):
    """Two GPU caches with the same full prefilled contents."""
    caches = []
    k, v, scores, tp, _ = W.random_cache(seed, w.B, w.Hkv, w.C, w.D, w.C, w.dtype, hh_frac=0.02)
    for _ in range(2):
        gc = H2OCache(w.B, w.Hq, w.Hkv, w.D, w.C, w.T, dtype=w.dtype, device=DEV)
        gc.k.copy_(to_dev(k))
        gc.v.copy_(to_dev(v))
        gc.scores.copy_(torch.from_numpy(scores).to(DEV))
        gc.token_pos.copy_(torch.from_numpy(tp).to(DEV))
        gc.n_occ = gc.pos = w.C
        caches.append(gc)
    return caches


def _compare(w, seed, wsum_null):
    ref, mine = _pair(w, seed)
    ch = W.random_chunk([seed, 1], w.B, w.Hq, w.Hkv, w.T, w.D, w.dtype, hh_frac=0.02)
    q, kn, vn = to_dev(ch["q"]), to_dev(ch["k"]), to_dev(ch["v"])
    o_ref, w_ref, s_ref = ref.new_outputs()
    api.h2o_chunk_step(ref.dims, ref.bufs(), w.C, w.C, q, kn, vn, o_ref, w_ref, s_ref, ref.ws)
    o, wsum, s = mine.new_outputs()
    wsum.fill_(-1.0)
    api.h2o_chunk_step_noalloc(mine.dims, mine.bufs(), w.C, w.C, q, kn, vn, o,
                               None if wsum_null else wsum, s)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), "output differs"
    if not wsum_null:
        assert torch.equal(wsum, w_ref), "summed weights differ"
    assert torch.equal(s, s_ref), "replay log differs"
    for name in ("k", "v", "scores", "token_pos"):
        a, b = getattr(mine, name), getattr(ref, name)
        if a.dtype == torch.bfloat16:
            a, b = a.view(torch.int16), b.view(torch.int16)
        assert torch.equal(a, b), f"cache {name} differs"


def test_noalloc_matches_chunk_step_twice_second_smaller():
    big = W.WORKLOADS[3].scaled(C=4096, T=512, name="noalloc_big")
    small = W.WORKLOADS[3].scaled(C=1024, T=4, name="noalloc_small")
    _compare(big, 91, wsum_null=False)
    _compare(small, 92, wsum_null=True)


def test_noalloc_rejects_workspace_beyond_the_array():
    # stored logits of a 4-token chunk on a 1M-slot cache need more than the
    # array; the call is rejected before any buffer is touched
    import ctypes
    dims = api.make_dims(1, 32, 8, 128, 1 << 20, 4)
    t = torch.zeros(16, dtype=torch.bfloat16, device=DEV)
    p = ctypes.c_void_p(t.data_ptr())
    bufs = api.H2OCacheBufs(p.value, p.value, None, None, None, None, p.value, p.value)
    st = api.lib().h2o_chunk_step_noalloc(ctypes.byref(dims), ctypes.byref(bufs), 1 << 20, 1 << 20, p, p, p, p,
                                          None, p, None)
    assert st == api.H2O_EWORKSPACE
