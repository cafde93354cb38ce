"""Plain fp64 CPU oracle for one H2O chunk step over a fixed-capacity KV cache.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
CPU-baseline leg of the benchmark may import this module.  The GPU library never
imports, links or calls it, and it shares no code with the GPU library.

What is computed, and where the pages define it
-----------------------------------------------
Pages: "Learning how to Forget: Fine-tuning for Long-Context Sparse Attention"
(paper text page, cited as [LF]) and the aimodeling.com article on the
KeysAndValues release (cited as [AM]).

* Cache buffers keys, values of shape (B, H_k, N_C, d_h), token_pos of shape
  (B, H_k, N_C); filled left to right up to N_C; grouped-query attention with
  H_q = H_k * q_g, q_g query heads per KV group ([LF] §3.1).
* Chunks of T tokens; per chunk B*H_k*T slots are overwritten by the new keys
  and values ([LF] §3.1).
* Softmax argument A = mask(d_h^{-1/2} Q K^T) and summed attention weights
  sum_i m[b,h,i,j] ([LF] §A.7, §3.1.1).  Causal masking by token position
  ([LF] §A.1).
* H2O score = cumulative sum of attention weights; the lowest-scoring entry is
  evicted ([AM]; [LF] §3.1.1).
* Replay log of the policy's decisions per chunk ([LF] §3.2).
* 8-bit and 4-bit cache buffers ([AM]; [LF] §2) -- the pages give no scheme.

Readings where the pages are silent or garbled
----------------------------------------------
R1 Step order is attend-then-evict: the chunk attends to the n_occ occupied
   slots (all visible, their tokens are older) plus its own keys causally; the
   eviction then uses scores that already include this chunk's sums.  With this
   order the token-position mask of [LF] §A.1 reduces to "cache fully visible,
   chunk causal".
R2 Summed weights are reduced over the q_g query heads of each KV group, so the
   score has one entry per (b, KV head, slot).
R3 Query head h uses KV head floor(h / q_g).
R4 Eviction candidates are the occupied slots only; all T new tokens enter.
R5 Bottom-T selection under the lexicographic key (score, slot index): ties go
   to the lower index.  New token t is written to the t-th smallest selected
   slot index, so the replay log row is the selected set in ascending order.
R6 A new slot's score is seeded with its own column sum from this chunk.
R7 A chunk either fits (n_occ + T <= C, fill) or meets a full cache
   (n_occ == C, evict); a chunk that would straddle capacity is rejected.
R8 Scale = d_h^{-1/2} given as an fp32 value; the oracle promotes it to fp64.
R9 The chunk attends to its own keys and values at input precision; they are
   quantised only when written into a quantised cache.
R11 Policy variants ([LF] §3.1.1).  h2o_orig ranks slot j of KV head h by
   the sum over batch rows of the per-row scores, so every batch row selects
   the same slots; the per-row scores are still kept.  h2o_norm ranks slot j
   by its score divided by its age t - t(b,h,j), with t the number of tokens
   processed once this chunk is attended (pos + T), i.e. the number of queries
   that have contributed to the score; the stored score stays cumulative.
R19 Gradients ([LF] §3.2, §A.10): the backward of the chunk attention is the
   exact derivative of attend_chunk's output with respect to q, the cache
   rows < n_occ and the chunk's keys and values (the summed weights carry no
   gradient); dK and dV of a KV group are summed over its query heads.
R10 Quantisers (fp32 operation sequences, IEEE round-to-nearest-even):
   int8 symmetric per slot:  a = max|x|;  s = fp16(fp32(a / 127));
        c = clamp(rne(fp32(x / fp32(s))), -127, 127);  x_hat = c * s
   int4 asymmetric per slot: z = fp16(min x);  s = fp16(fp32(fp32(max x - min x) / 15));
        c = clamp(rne(fp32(fp32(x - fp32(z)) / fp32(s))), 0, 15);  x_hat = c * s + z
   s == 0 gives all-zero codes.  Two 4-bit codes per byte, element 2k in the
   low nibble.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "attend_chunk",
    "update_scores",
    "bottom_t",
    "selection_key",
    "POLICIES",
    "quantize_int8",
    "quantize_int4",
    "dequantize_int8",
    "dequantize_int4",
    "pack_nibbles",
    "unpack_nibbles",
    "OracleCache",
]

NEG_INF = -np.inf


# --------------------------------------------------------------------------
# Attention with summed weights
# --------------------------------------------------------------------------

def attend_chunk(q, k_cache, v_cache, n_occ, k_new, v_new, scale, row_block=256):
    """Exact softmax attention of one chunk plus summed attention weights.

    [LF] §A.7: A = mask(d_h^{-1/2} Q K^T), m = softmax(A) along keys, Y = m V,
    summed weights sum_i m[b,h,i,j].  [LF] §3.1: GQA grouping.  Readings R1-R3.

    Args (all float64 numpy arrays holding the stored values exactly):
      q        (B, Hq, T, D)
      k_cache  (B, Hkv, >= n_occ, D)  dequantised cache keys; slots < n_occ used
      v_cache  (B, Hkv, >= n_occ, D)
      k_new    (B, Hkv, T, D), v_new (B, Hkv, T, D)
      scale    python float (the fp32 scale promoted to fp64)

    Returns:
      out (B, Hq, T, D)     attention output
      w   (B, Hkv, n_occ+T) weights summed over queries and the heads of a group
      lse (B, Hq, T)        natural-log normaliser log sum_j exp(A_ij)
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, T, D = q.shape
    Hkv = k_new.shape[1]
    assert Hq % Hkv == 0, "Hq must be a multiple of Hkv"
    qg = Hq // Hkv
    n_keys = n_occ + T
    out = np.zeros((B, Hq, T, D))
    w = np.zeros((B, Hkv, n_keys))
    lse = np.zeros((B, Hq, T))
    t_new = np.arange(T)
    for b in range(B):
        for g in range(Hkv):
            keys = np.concatenate([k_cache[b, g, :n_occ], k_new[b, g]], axis=0)
            vals = np.concatenate([v_cache[b, g, :n_occ], v_new[b, g]], axis=0)
            for hh in range(qg):
                h = g * qg + hh
                for i0 in range(0, T, row_block):
                    i1 = min(T, i0 + row_block)
                    logits = scale * (q[b, h, i0:i1] @ keys.T)
                    # cache slots are all visible; new key t' is visible to query i iff t' <= i
                    hidden = t_new[None, :] > np.arange(i0, i1)[:, None]
                    logits[:, n_occ:][hidden] = NEG_INF
                    row_max = logits.max(axis=1, keepdims=True)
                    e = np.exp(logits - row_max)
                    row_sum = e.sum(axis=1, keepdims=True)
                    m = e / row_sum
                    out[b, h, i0:i1] = m @ vals
                    w[b, g] += m.sum(axis=0)
                    lse[b, h, i0:i1] = (row_max + np.log(row_sum))[:, 0]
    return out, w, lse


# --------------------------------------------------------------------------
# Score update and bottom-T selection
# --------------------------------------------------------------------------

def attend_backward(q, k_cache, v_cache, n_occ, k_new, v_new, scale, dout):
    """Gradients of the chunk attention of attend_chunk for an upstream
    gradient dout = dL/d(out).

    [LF] §3.2: the fine-tuning pass obtains gradients by reverse-mode
    differentiation through each chunk's SDPA call; [LF] §A.10: the attention
    interface that returns summed weights also has a backward.  The summed
    weights only steer eviction and carry no gradient.  Reading R19.

    With P = softmax of the masked scaled logits (attend_chunk), per query
    row r of a KV group and key j of the group:
      dV_j  = sum_r P_rj dO_r                 (summed over the group's heads)
      dP_rj = <dO_r, v_j>
      dS_rj = P_rj (dP_rj - sum_j' P_rj' dP_rj')
      dQ_r  = scale sum_j dS_rj k_j
      dK_j  = scale sum_r dS_rj q_r           (summed over the group's heads)
    Masked pairs have P = 0 and contribute nothing.  (The row term
    sum_j' P_rj' dP_rj' equals <dO_r, O_r>.)

    Returns float64 arrays dq (B, Hq, T, D), dk_cache, dv_cache
    (B, Hkv, n_occ, D), dk_new, dv_new (B, Hkv, T, D).
    """
    q = np.asarray(q, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, Hq, T, D = q.shape
    Hkv = k_new.shape[1]
    qg = Hq // Hkv
    n_keys = n_occ + T
    dq = np.zeros((B, Hq, T, D))
    dk = np.zeros((B, Hkv, n_keys, D))
    dv = np.zeros((B, Hkv, n_keys, D))
    hidden = np.arange(T)[None, :] > np.arange(T)[:, None]  # new key t' hidden from query i < t'
    for b in range(B):
        for g in range(Hkv):
            keys = np.concatenate([k_cache[b, g, :n_occ], k_new[b, g]], axis=0)
            vals = np.concatenate([v_cache[b, g, :n_occ], v_new[b, g]], axis=0)
            for hh in range(qg):
                h = g * qg + hh
                logits = scale * (q[b, h] @ keys.T)
                logits[:, n_occ:][hidden] = NEG_INF
                e = np.exp(logits - logits.max(axis=1, keepdims=True))
                p = e / e.sum(axis=1, keepdims=True)
                dp = dout[b, h] @ vals.T
                row = (p * dp).sum(axis=1, keepdims=True)
                ds = p * (dp - row)
                dq[b, h] = scale * (ds @ keys)
                dk[b, g] += scale * (ds.T @ q[b, h])
                dv[b, g] += p.T @ dout[b, h]
    return dq, dk[:, :, :n_occ], dv[:, :, :n_occ], dk[:, :, n_occ:], dv[:, :, n_occ:]


def update_scores(phi, w, n_occ, C, T):
    """Add this chunk's summed weights to the running H2O scores of the
    occupied slots ([AM]: cumulative sums; [LF] §3.1.1).

    Returns the updated copy; slots >= n_occ are left as they were.
    """
    phi = np.array(phi, dtype=np.float64, copy=True)
    phi[..., :n_occ] += w[..., :n_occ]
    return phi


POLICIES = ("h2o", "h2o_norm", "h2o_orig")


def selection_key(phi_updated, token_pos, pos, T, policy="h2o"):
    """The value the occupied slots are ranked by when the cache is full
    ([LF] §3.1.1, reading R11), shape (B, Hkv, C).

    h2o:      the cumulative score itself.
    h2o_norm: score / (t - t(b,h,j)) with t = pos + T.
    h2o_orig: sum over b of the scores, the same for every b.
    """
    phi = np.asarray(phi_updated, dtype=np.float64)
    if policy == "h2o":
        return phi.copy()
    if policy == "h2o_norm":
        age = (pos + T) - np.asarray(token_pos, dtype=np.float64)
        return phi / age
    if policy == "h2o_orig":
        tot = phi.sum(axis=0, keepdims=True)
        return np.broadcast_to(tot, phi.shape).copy()
    raise ValueError(f"unknown policy {policy!r}")


def bottom_t(phi_updated, n_occ, C, T):
    """Slots that receive the chunk's T tokens (readings R4, R5, R7).

    Fill (n_occ + T <= C): slots n_occ .. n_occ+T-1 (left to right, [LF] §3.1).
    Evict (n_occ == C): the T smallest entries under (key, index), returned in
    ascending index order; the key is the updated score, or the policy's
    selection_key.
    """
    B, Hkv = phi_updated.shape[:2]
    if n_occ + T <= C:
        row = np.arange(n_occ, n_occ + T, dtype=np.int64)
        return np.broadcast_to(row, (B, Hkv, T)).copy()
    if n_occ != C:
        raise ValueError("chunk straddles capacity (n_occ < C < n_occ + T)")
    if T > C:
        raise ValueError("chunk longer than the cache")
    slots = np.empty((B, Hkv, T), dtype=np.int64)
    idx = np.arange(C)
    for b in range(B):
        for g in range(Hkv):
            order = np.lexsort((idx, phi_updated[b, g, :C]))
            slots[b, g] = np.sort(order[:T])
    return slots


# --------------------------------------------------------------------------
# Quantisers (reading R10), in numpy float32 / float16 arithmetic
# --------------------------------------------------------------------------

def quantize_int8(x):
    """Symmetric 8-bit codes per row (last axis) with an fp16 scale.

    x: float32 array (..., D).  Returns (codes int8 (..., D), scale float16 (...)).
    """
    x = np.asarray(x, dtype=np.float32)
    a = np.max(np.abs(x), axis=-1)
    s16 = (a / np.float32(127.0)).astype(np.float16)
    s32 = s16.astype(np.float32)[..., None]
    q = np.zeros_like(x)
    np.divide(x, s32, out=q, where=(s32 != 0))
    c = np.clip(np.rint(q), -127, 127).astype(np.int8)
    return c, s16


def quantize_int4(x):
    """Asymmetric 4-bit codes per row (last axis) with fp16 scale and zero point.

    x: float32 array (..., D), D even.  Returns (packed uint8 (..., D/2),
    scale float16 (...), zero float16 (...)).
    """
    x = np.asarray(x, dtype=np.float32)
    lo = np.min(x, axis=-1)
    hi = np.max(x, axis=-1)
    z16 = lo.astype(np.float16)
    span = (hi - lo).astype(np.float32)
    s16 = (span / np.float32(15.0)).astype(np.float16)
    z32 = z16.astype(np.float32)[..., None]
    s32 = s16.astype(np.float32)[..., None]
    shifted = (x - z32).astype(np.float32)
    q = np.zeros_like(x)
    np.divide(shifted, s32, out=q, where=(s32 != 0))
    c = np.clip(np.rint(q), 0, 15).astype(np.uint8)
    return pack_nibbles(c), s16, z16


def pack_nibbles(c):
    """Two 4-bit codes per byte; element 2k in the low nibble."""
    c = np.asarray(c, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(p):
    p = np.asarray(p, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def dequantize_int8(codes, scale):
    return codes.astype(np.float64) * scale.astype(np.float64)[..., None]


def dequantize_int4(packed, scale, zero):
    c = unpack_nibbles(packed).astype(np.float64)
    return c * scale.astype(np.float64)[..., None] + zero.astype(np.float64)[..., None]


# --------------------------------------------------------------------------
# One layer's cache state and the full chunk step
# --------------------------------------------------------------------------

class OracleCache:
    """State of one layer's fixed-capacity cache, updated one chunk at a time.

    fmt: "native" (values stored at input precision), "int8" or "int4".
    Scores are held in fp64; token_pos starts at -1 for empty slots.
    """

    def __init__(self, B, Hq, Hkv, D, C, fmt="native", scale=None, policy="h2o"):
        assert Hq % Hkv == 0
        self.B, self.Hq, self.Hkv, self.D, self.C = B, Hq, Hkv, D, C
        self.fmt = fmt
        if policy not in POLICIES:
            raise ValueError(f"unknown policy {policy!r}")
        self.policy = policy
        self.scale = float(np.float32(1.0 / np.sqrt(D))) if scale is None else float(scale)
        self.k = np.zeros((B, Hkv, C, D))      # values attended (dequantised for int formats)
        self.v = np.zeros((B, Hkv, C, D))
        self.phi = np.zeros((B, Hkv, C))
        self.token_pos = np.full((B, Hkv, C), -1, dtype=np.int64)
        self.n_occ = 0
        self.pos = 0
        if fmt == "int8":
            self.k_codes = np.zeros((B, Hkv, C, D), np.int8)
            self.v_codes = np.zeros((B, Hkv, C, D), np.int8)
        elif fmt == "int4":
            self.k_codes = np.zeros((B, Hkv, C, D // 2), np.uint8)
            self.v_codes = np.zeros((B, Hkv, C, D // 2), np.uint8)
            self.k_zero = np.zeros((B, Hkv, C), np.float16)
            self.v_zero = np.zeros((B, Hkv, C), np.float16)
        elif fmt != "native":
            raise ValueError(fmt)
        if fmt in ("int8", "int4"):
            self.k_scale = np.zeros((B, Hkv, C), np.float16)
            self.v_scale = np.zeros((B, Hkv, C), np.float16)

    # -- writing rows ----------------------------------------------------
    def _write_rows(self, b, g, slots, k_rows, v_rows):
        if self.fmt == "native":
            self.k[b, g, slots] = k_rows
            self.v[b, g, slots] = v_rows
            return
        k32 = k_rows.astype(np.float32)
        v32 = v_rows.astype(np.float32)
        if self.fmt == "int8":
            kc, ks = quantize_int8(k32)
            vc, vs = quantize_int8(v32)
            self.k_codes[b, g, slots], self.k_scale[b, g, slots] = kc, ks
            self.v_codes[b, g, slots], self.v_scale[b, g, slots] = vc, vs
            self.k[b, g, slots] = dequantize_int8(kc, ks)
            self.v[b, g, slots] = dequantize_int8(vc, vs)
        else:
            kc, ks, kz = quantize_int4(k32)
            vc, vs, vz = quantize_int4(v32)
            self.k_codes[b, g, slots], self.k_scale[b, g, slots], self.k_zero[b, g, slots] = kc, ks, kz
            self.v_codes[b, g, slots], self.v_scale[b, g, slots], self.v_zero[b, g, slots] = vc, vs, vz
            self.k[b, g, slots] = dequantize_int4(kc, ks, kz)
            self.v[b, g, slots] = dequantize_int4(vc, vs, vz)

    # -- one chunk step --------------------------------------------------
    def step(self, q, k_new, v_new):
        """Attend, accumulate scores, select, log and overwrite (readings R1-R9).

        q (B,Hq,T,D), k_new/v_new (B,Hkv,T,D): float64 arrays of the input values.
        Returns dict(out, w, lse, slots, phi_updated, rank_key) where phi_updated
        holds the scores after accumulation and before the selected slots are
        re-seeded, and rank_key the values the slots were ranked by.
        """
        T = q.shape[2]
        C, n_occ = self.C, self.n_occ
        if not (n_occ + T <= C or n_occ == C):
            raise ValueError("chunk straddles capacity")
        out, w, lse = attend_chunk(q, self.k, self.v, n_occ, k_new, v_new, self.scale)
        phi_upd = update_scores(self.phi, w, n_occ, C, T)
        key = phi_upd
        if n_occ == C:
            key = selection_key(phi_upd, self.token_pos, self.pos, T, self.policy)
        slots = bottom_t(key, n_occ, C, T)
        self.phi = phi_upd.copy()
        for b in range(self.B):
            for g in range(self.Hkv):
                r = slots[b, g]
                self._write_rows(b, g, r, k_new[b, g], v_new[b, g])
                self.phi[b, g, r] = w[b, g, n_occ:n_occ + T]
                self.token_pos[b, g, r] = self.pos + np.arange(T)
        self.n_occ = min(n_occ + T, C)
        self.pos += T
        return dict(out=out, w=w, lse=lse, slots=slots, phi_updated=phi_upd, rank_key=key)

    def replay_step(self, q, k_new, v_new, slots):
        """Replay a logged decision ([LF] §3.2: replay caches act like normal
        caches but take their eviction decisions from the log): attend as in
        step(), write the chunk into the logged slots (quantising for 8/4-bit
        caches) and set their token positions.  No score is computed or kept.

        slots: integer array (B, Hkv, T), one replay-log row per (b, g).
        Returns out.
        """
        T = q.shape[2]
        C, n_occ = self.C, self.n_occ
        if not (n_occ + T <= C or n_occ == C):
            raise ValueError("chunk straddles capacity")
        out, _, _ = attend_chunk(q, self.k, self.v, n_occ, k_new, v_new, self.scale)
        for b in range(self.B):
            for g in range(self.Hkv):
                r = np.asarray(slots[b, g], dtype=np.int64)
                self._write_rows(b, g, r, k_new[b, g], v_new[b, g])
                self.token_pos[b, g, r] = self.pos + np.arange(T)
        self.n_occ = min(n_occ + T, C)
        self.pos += T
        return out
