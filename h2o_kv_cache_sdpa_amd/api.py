"""ctypes binding of libh2o.so (declared in include/h2o.h).

Argument marshalling only: every step of the chunk step runs in the HIP
library.  Tensors are torch tensors on the GPU (PyTorch supplies device memory
and streams); their data pointers and the current stream's handle are passed
through unchanged.  If the library is missing, loading raises -- there is no
fallback.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# H2O_DEBUG_LIB=1 selects the debug build (device index checks on).
LIB_PATH = os.path.join(PKG, "libh2o_debug.so" if os.environ.get("H2O_DEBUG_LIB") == "1" else "libh2o.so")

H2O_OK, H2O_EINVAL, H2O_EUNSUPPORTED, H2O_EWORKSPACE, H2O_EHIP = 0, -1, -2, -3, -4
H2O_F32, H2O_BF16 = 0, 1
H2O_CACHE_NATIVE, H2O_CACHE_INT8, H2O_CACHE_INT4 = 0, 1, 2
H2O_POLICY_H2O = 0

DTYPES = {"f32": H2O_F32, "bf16": H2O_BF16}
FORMATS = {"native": H2O_CACHE_NATIVE, "int8": H2O_CACHE_INT8, "int4": H2O_CACHE_INT4}

EXPORTS = (
    "h2o_abi_version", "h2o_status_str", "h2o_last_hip_error", "h2o_workspace_bytes",
    "h2o_sdpa_scoresum", "h2o_evict_topk", "kv_scatter", "kv_quant_pack",
    "kv_dequant_unpack", "h2o_chunk_step", "h2o_chunk_step_noalloc", "h2o_replay_step",
    "h2o_sdpa_backward",
    "h2o_profile_enable", "h2o_profile_read",
    "h2o_profile_reset",
)
KERNEL_KINDS = ("attn_a", "attn_b", "evict", "kv_write", "attn_combine", "bwd_rows", "bwd_dq", "bwd_dkdv")


class H2ODims(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("D", ctypes.c_int32), ("C", ctypes.c_int32), ("T", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("cache_fmt", ctypes.c_int32), ("policy", ctypes.c_int32),
        ("scale", ctypes.c_float),
    ]


class H2OCacheBufs(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("k_zero", ctypes.c_void_p), ("v_zero", ctypes.c_void_p),
        ("scores", ctypes.c_void_p), ("token_pos", ctypes.c_void_p),
    ]


class H2OError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        msg = f"{fn} failed: {status_str(status)} ({status})"
        if status == H2O_EHIP:
            msg += f", hipError {lib().h2o_last_hip_error()}"
        super().__init__(msg)


_lib = None


def lib():
    """Load libh2o.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} not built: run __graft_entry__.build() "
                           "or python -m h2o_kv_cache_sdpa_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    P, S, I32, I64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
    pd, pc = ctypes.POINTER(H2ODims), ctypes.POINTER(H2OCacheBufs)
    L.h2o_abi_version.restype = ctypes.c_int
    L.h2o_abi_version.argtypes = []
    L.h2o_status_str.restype = ctypes.c_char_p
    L.h2o_status_str.argtypes = [ctypes.c_int]
    L.h2o_last_hip_error.restype = ctypes.c_int
    L.h2o_last_hip_error.argtypes = []
    L.h2o_workspace_bytes.restype = S
    L.h2o_workspace_bytes.argtypes = [pd]
    L.h2o_sdpa_scoresum.restype = ctypes.c_int
    L.h2o_sdpa_scoresum.argtypes = [pd, pc, I32, P, P, P, P, P, P, P, S, P]
    L.h2o_evict_topk.restype = ctypes.c_int
    L.h2o_evict_topk.argtypes = [pd, pc, I32, I64, P, P, P, S, P]
    for name in ("kv_scatter", "kv_quant_pack"):
        f = getattr(L, name)
        f.restype = ctypes.c_int
        f.argtypes = [pd, pc, P, P, P, P]
    L.kv_dequant_unpack.restype = ctypes.c_int
    L.kv_dequant_unpack.argtypes = [pd, pc, I32, P, P, P]
    L.h2o_chunk_step.restype = ctypes.c_int
    L.h2o_chunk_step.argtypes = [pd, pc, I32, I64, P, P, P, P, P, P, P, S, P]
    L.h2o_chunk_step_noalloc.restype = ctypes.c_int
    L.h2o_chunk_step_noalloc.argtypes = [pd, pc, I32, I64, P, P, P, P, P, P, P]
    L.h2o_replay_step.restype = ctypes.c_int
    L.h2o_replay_step.argtypes = [pd, pc, I32, I64, P, P, P, P, P, P, S, P]
    L.h2o_sdpa_backward.restype = ctypes.c_int
    L.h2o_sdpa_backward.argtypes = [pd, pc, I32] + [P] * 10 + [P, S, P]
    L.h2o_profile_enable.restype = ctypes.c_int
    L.h2o_profile_enable.argtypes = [ctypes.c_int]
    L.h2o_profile_read.restype = ctypes.c_int
    L.h2o_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64),
                                   ctypes.c_int]
    L.h2o_profile_reset.restype = ctypes.c_int
    L.h2o_profile_reset.argtypes = []
    _lib = L
    return L


def status_str(status):
    return lib().h2o_status_str(int(status)).decode()


POLICIES = {"h2o": 0, "h2o_norm": 1, "h2o_orig": 2}


def make_dims(B, Hq, Hkv, D, C, T, dtype="bf16", cache_fmt="native", scale=0.0, policy=0):
    return H2ODims(B, Hq, Hkv, D, C, T, DTYPES.get(dtype, dtype), FORMATS.get(cache_fmt, cache_fmt),
                   POLICIES.get(policy, policy), float(scale))


def workspace_bytes(dims):
    return int(lib().h2o_workspace_bytes(ctypes.byref(dims)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _torch():
    import torch
    return torch


def _need(t, what, numel, dtypes, required=True):
    """A tensor handed to the library must live on the GPU, be contiguous and
    have the element type and element count the dimensions call for: the
    library only sees its address."""
    if t is None:
        if required:
            raise ValueError(f"{what} is required")
        return
    if not t.is_cuda:
        raise ValueError(f"{what} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if t.dtype not in dtypes:
        raise ValueError(f"{what} has dtype {t.dtype}, expected one of {dtypes}")
    if t.numel() != numel:
        raise ValueError(f"{what} has {t.numel()} elements, expected {numel}")


def _io_dtype(dims):
    torch = _torch()
    return (torch.float32,) if dims.dtype == H2O_F32 else (torch.bfloat16,)


def _check_chunk(dims, q, k_new, v_new, out=None, need_out=True):
    torch = _torch()
    dt = _io_dtype(dims)
    B, Hq, Hkv, D, T = dims.B, dims.Hq, dims.Hkv, dims.D, dims.T
    _need(q, "q", B * Hq * T * D, dt)
    _need(k_new, "k_new", B * Hkv * T * D, dt)
    _need(v_new, "v_new", B * Hkv * T * D, dt)
    if need_out:
        _need(out, "out", B * Hq * T * D, dt)
    return torch


def cache_struct(k, v, scores=None, token_pos=None, k_scale=None, v_scale=None, k_zero=None,
                 v_zero=None, dims=None):
    """Pointers of one cache's state tensors; with `dims`, each tensor given
    is checked against the cache layout first."""
    if dims is not None:
        torch = _torch()
        B, Hkv, C, D = dims.B, dims.Hkv, dims.C, dims.D
        if dims.cache_fmt == H2O_CACHE_NATIVE:
            kv_n, kv_dt = B * Hkv * C * D, _io_dtype(dims)
        elif dims.cache_fmt == H2O_CACHE_INT8:
            kv_n, kv_dt = B * Hkv * C * D, (torch.int8,)
        else:
            kv_n, kv_dt = B * Hkv * C * D // 2, (torch.uint8,)
        _need(k, "cache k", kv_n, kv_dt)
        _need(v, "cache v", kv_n, kv_dt)
        for name, t in (("k_scale", k_scale), ("v_scale", v_scale), ("k_zero", k_zero), ("v_zero", v_zero)):
            _need(t, name, B * Hkv * C, (torch.float16,), required=False)
        _need(scores, "scores", B * Hkv * C, (torch.float32,), required=False)
        _need(token_pos, "token_pos", B * Hkv * C, (torch.int32,), required=False)
    f = lambda t: None if t is None else t.data_ptr()
    return H2OCacheBufs(f(k), f(v), f(k_scale), f(v_scale), f(k_zero), f(v_zero), f(scores),
                        f(token_pos))


def _check(fn, st):
    if st != H2O_OK:
        raise H2OError(fn, st)


def _check_ws(ws):
    torch = _torch()
    _need(ws, "ws", ws.numel() if ws is not None else 0, (torch.uint8,))


def h2o_sdpa_scoresum(dims, cache, n_occ, q, k_new, v_new, out, wsum, lse, ws, stream=None):
    torch = _check_chunk(dims, q, k_new, v_new, out)
    _need(wsum, "wsum", dims.B * dims.Hkv * (int(n_occ) + dims.T), (torch.float32,))
    _need(lse, "lse", dims.B * dims.Hq * dims.T, (torch.float32,), required=False)
    _check_ws(ws)
    st = lib().h2o_sdpa_scoresum(ctypes.byref(dims), ctypes.byref(cache), int(n_occ), _ptr(q),
                                 _ptr(k_new), _ptr(v_new), _ptr(out), _ptr(wsum), _ptr(lse),
                                 _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check("h2o_sdpa_scoresum", st)


def h2o_evict_topk(dims, cache, n_occ, pos, wsum, slot_log, ws=None, stream=None):
    torch = _torch()
    _need(wsum, "wsum", dims.B * dims.Hkv * (int(n_occ) + dims.T), (torch.float32,))
    _need(slot_log, "slot_log", dims.B * dims.Hkv * dims.T, (torch.int32,))
    if ws is not None:
        _check_ws(ws)
    nb = 0 if ws is None else ws.numel() * ws.element_size()
    st = lib().h2o_evict_topk(ctypes.byref(dims), ctypes.byref(cache), int(n_occ), int(pos),
                              _ptr(wsum), _ptr(slot_log), _ptr(ws), nb, _stream(stream))
    _check("h2o_evict_topk", st)


def kv_scatter(dims, cache, k_new, v_new, slot_log, stream=None):
    torch = _torch()
    dt = _io_dtype(dims)
    _need(k_new, "k_new", dims.B * dims.Hkv * dims.T * dims.D, dt)
    _need(v_new, "v_new", dims.B * dims.Hkv * dims.T * dims.D, dt)
    _need(slot_log, "slot_log", dims.B * dims.Hkv * dims.T, (torch.int32,))
    st = lib().kv_scatter(ctypes.byref(dims), ctypes.byref(cache), _ptr(k_new), _ptr(v_new),
                          _ptr(slot_log), _stream(stream))
    _check("kv_scatter", st)


def kv_quant_pack(dims, cache, k_new, v_new, slot_log, stream=None):
    torch = _torch()
    dt = _io_dtype(dims)
    _need(k_new, "k_new", dims.B * dims.Hkv * dims.T * dims.D, dt)
    _need(v_new, "v_new", dims.B * dims.Hkv * dims.T * dims.D, dt)
    _need(slot_log, "slot_log", dims.B * dims.Hkv * dims.T, (torch.int32,))
    st = lib().kv_quant_pack(ctypes.byref(dims), ctypes.byref(cache), _ptr(k_new), _ptr(v_new),
                             _ptr(slot_log), _stream(stream))
    _check("kv_quant_pack", st)


def kv_dequant_unpack(dims, cache, n_slots, k_out, v_out, stream=None):
    torch = _torch()
    for name, t in (("k_out", k_out), ("v_out", v_out)):
        _need(t, name, dims.B * dims.Hkv * int(n_slots) * dims.D, (torch.float32,))
    st = lib().kv_dequant_unpack(ctypes.byref(dims), ctypes.byref(cache), int(n_slots),
                                 _ptr(k_out), _ptr(v_out), _stream(stream))
    _check("kv_dequant_unpack", st)


def h2o_chunk_step(dims, cache, n_occ, pos, q, k_new, v_new, out, wsum, slot_log, ws, stream=None,
                   check=True):
    """check=False skips the tensor checks (for a timing loop whose tensors
    have already been checked once)."""
    if check:
        torch = _check_chunk(dims, q, k_new, v_new, out)
        _need(wsum, "wsum", dims.B * dims.Hkv * (int(n_occ) + dims.T), (torch.float32,), required=False)
        _need(slot_log, "slot_log", dims.B * dims.Hkv * dims.T, (torch.int32,))
        _check_ws(ws)
    st = lib().h2o_chunk_step(ctypes.byref(dims), ctypes.byref(cache), int(n_occ), int(pos),
                              _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out), _ptr(wsum),
                              _ptr(slot_log), _ptr(ws), ws.numel() * ws.element_size(),
                              _stream(stream))
    _check("h2o_chunk_step", st)


def h2o_chunk_step_noalloc(dims, cache, n_occ, pos, q, k_new, v_new, out, wsum, slot_log, stream=None):
    torch = _check_chunk(dims, q, k_new, v_new, out)
    _need(wsum, "wsum", dims.B * dims.Hkv * (int(n_occ) + dims.T), (torch.float32,), required=False)
    _need(slot_log, "slot_log", dims.B * dims.Hkv * dims.T, (torch.int32,))
    st = lib().h2o_chunk_step_noalloc(ctypes.byref(dims), ctypes.byref(cache), int(n_occ), int(pos),
                                      _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out), _ptr(wsum),
                                      _ptr(slot_log), _stream(stream))
    _check("h2o_chunk_step_noalloc", st)


def h2o_replay_step(dims, cache, n_occ, pos, q, k_new, v_new, out, slot_log, ws, stream=None, check=True):
    if check:
        torch = _check_chunk(dims, q, k_new, v_new, out)
        _need(slot_log, "slot_log", dims.B * dims.Hkv * dims.T, (torch.int32,))
        _check_ws(ws)
    st = lib().h2o_replay_step(ctypes.byref(dims), ctypes.byref(cache), int(n_occ), int(pos),
                               _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out), _ptr(slot_log),
                               _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check("h2o_replay_step", st)


def h2o_sdpa_backward(dims, cache, n_occ, q, k_new, v_new, lse, dout, dq, dk_cache, dv_cache,
                      dk_new, dv_new, ws, stream=None):
    torch = _check_chunk(dims, q, k_new, v_new, need_out=False)
    B, Hq, Hkv, D, C, T = dims.B, dims.Hq, dims.Hkv, dims.D, dims.C, dims.T
    _need(lse, "lse", B * Hq * T, (torch.float32,))
    _need(dout, "dout", B * Hq * T * D, _io_dtype(dims))
    _need(dq, "dq", B * Hq * T * D, (torch.float32,))
    for name, t in (("dk_cache", dk_cache), ("dv_cache", dv_cache)):
        _need(t, name, B * Hkv * C * D, (torch.float32,), required=int(n_occ) > 0)
    for name, t in (("dk_new", dk_new), ("dv_new", dv_new)):
        _need(t, name, B * Hkv * T * D, (torch.float32,))
    _check_ws(ws)
    st = lib().h2o_sdpa_backward(ctypes.byref(dims), ctypes.byref(cache), int(n_occ), _ptr(q),
                                 _ptr(k_new), _ptr(v_new), _ptr(lse), _ptr(dout), _ptr(dq),
                                 _ptr(dk_cache), _ptr(dv_cache), _ptr(dk_new), _ptr(dv_new),
                                 _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check("h2o_sdpa_backward", st)


def profile_enable(on=True):
    _check("h2o_profile_enable", lib().h2o_profile_enable(1 if on else 0))


def profile_reset():
    _check("h2o_profile_reset", lib().h2o_profile_reset())


def profile_read():
    """{kind: (total_ms, launches)} for the kernels timed since the last reset."""
    n = len(KERNEL_KINDS)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _check("h2o_profile_read", lib().h2o_profile_read(ms, cnt, n))
    return {k: (ms[i], cnt[i]) for i, k in enumerate(KERNEL_KINDS)}
