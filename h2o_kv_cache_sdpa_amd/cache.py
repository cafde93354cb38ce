"""H2OCache: one layer's fixed-capacity cache as torch device tensors.

PyTorch supplies the device memory and the stream; every step runs in
libh2o.so through the C ABI (``api``).  Host-side state is only the occupancy
``n_occ`` and the absolute position ``pos`` of the next chunk.
"""

from __future__ import annotations

import torch

from . import api

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


class H2OCache:
    def __init__(self, B, Hq, Hkv, D, C, T, dtype="bf16", cache_fmt="native", scale=0.0,
                 device="cuda", track_positions=True, policy="h2o"):
        self.B, self.Hq, self.Hkv, self.D, self.C, self.T = B, Hq, Hkv, D, C, T
        self.dtype, self.cache_fmt, self.policy = dtype, cache_fmt, policy
        self.dims = api.make_dims(B, Hq, Hkv, D, C, T, dtype, cache_fmt, scale, policy)
        self.device = torch.device(device)
        z = dict(device=self.device)
        self.k_scale = self.v_scale = self.k_zero = self.v_zero = None
        if cache_fmt == "native":
            self.k = torch.zeros(B, Hkv, C, D, dtype=_TORCH_DTYPE[dtype], **z)
            self.v = torch.zeros_like(self.k)
        elif cache_fmt == "int8":
            self.k = torch.zeros(B, Hkv, C, D, dtype=torch.int8, **z)
            self.v = torch.zeros_like(self.k)
        elif cache_fmt == "int4":
            self.k = torch.zeros(B, Hkv, C, D // 2, dtype=torch.uint8, **z)
            self.v = torch.zeros_like(self.k)
        else:
            raise ValueError(cache_fmt)
        if cache_fmt != "native":
            self.k_scale = torch.zeros(B, Hkv, C, dtype=torch.float16, **z)
            self.v_scale = torch.zeros_like(self.k_scale)
        if cache_fmt == "int4":
            self.k_zero = torch.zeros(B, Hkv, C, dtype=torch.float16, **z)
            self.v_zero = torch.zeros_like(self.k_zero)
        self.scores = torch.zeros(B, Hkv, C, dtype=torch.float32, **z)
        self.token_pos = torch.full((B, Hkv, C), -1, dtype=torch.int32, **z) if track_positions else None
        nbytes = api.workspace_bytes(self.dims)
        if nbytes == 0:
            raise ValueError("invalid cache dimensions")
        self.ws = torch.empty(nbytes, dtype=torch.uint8, **z)
        self.n_occ = 0
        self.pos = 0

    def bufs(self):
        return api.cache_struct(self.k, self.v, self.scores, self.token_pos, self.k_scale,
                                self.v_scale, self.k_zero, self.v_zero, dims=self.dims)

    def new_outputs(self, n_occ=None):
        n = self.n_occ if n_occ is None else n_occ
        z = dict(device=self.device)
        out = torch.empty(self.B, self.Hq, self.T, self.D, dtype=_TORCH_DTYPE[self.dtype], **z)
        wsum = torch.empty(self.B, self.Hkv, n + self.T, dtype=torch.float32, **z)
        slot_log = torch.empty(self.B, self.Hkv, self.T, dtype=torch.int32, **z)
        return out, wsum, slot_log

    def step(self, q, k_new, v_new, out=None, wsum=None, slot_log=None, stream=None):
        """One chunk step; returns (out, wsum, slot_log)."""
        o, w, s = self.new_outputs()
        out = o if out is None else out
        wsum = w if wsum is None else wsum
        slot_log = s if slot_log is None else slot_log
        bufs = self.bufs()
        api.h2o_chunk_step(self.dims, bufs, self.n_occ, self.pos, q, k_new, v_new, out, wsum,
                           slot_log, self.ws, stream)
        self.n_occ = min(self.n_occ + self.T, self.C)
        self.pos += self.T
        return out, wsum, slot_log

    def replay_step(self, q, k_new, v_new, slot_log, out=None, stream=None):
        """Attend and overwrite the slots of a logged decision (no scoring);
        returns out."""
        if out is None:
            out = self.new_outputs()[0]
        api.h2o_replay_step(self.dims, self.bufs(), self.n_occ, self.pos, q, k_new, v_new, out,
                            slot_log, self.ws, stream)
        self.n_occ = min(self.n_occ + self.T, self.C)
        self.pos += self.T
        return out
