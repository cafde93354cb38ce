/*
 * h2o.h -- C ABI of libh2o.so: one chunk step of H2O sparse attention over a
 * fixed-capacity KV cache, on one AMD Instinct MI355X (gfx950).
 *
 * The operation ("Learning how to Forget: Fine-tuning for Long-Context Sparse
 * Attention", paper text page, §3.1, §3.1.1, §3.2, §A.1, §A.7; aimodeling.com
 * article on the KeysAndValues release):
 *
 *   A chunk of T queries under grouped-query attention (H_q = H_kv * q_g; query
 *   head h reads KV head floor(h / q_g)) attends to the n_occ occupied slots of
 *   a cache of capacity C plus its own T keys, causally.  The step returns the
 *   attention output and the attention weights summed over the chunk's queries
 *   and over the q_g query heads of each KV group, for every occupied slot and
 *   chunk position.  It then adds those sums to the running H2O scores, picks
 *   the slots that receive the chunk (left-to-right fill while the cache has
 *   room; otherwise the T lowest-scoring slots, ties to the lower slot index),
 *   logs them (replay log), overwrites them with the chunk's keys and values
 *   (quantising them for 8-bit / 4-bit caches) and seeds their scores with
 *   their own summed weights.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers to contiguous row-major memory,
 *     16-byte aligned; the caller allocates and owns all of them and keeps them
 *     alive until the work on `stream` has completed.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *     is enqueued asynchronously; no entry point synchronises, allocates or
 *     frees device memory, or keeps a pointer after it returns.
 *   - Arguments are validated on the host before anything is enqueued; on an
 *     error nothing is enqueued and a negative h2o_status is returned.
 *   - Results are deterministic bit for bit (fixed-order reductions, no
 *     floating-point atomics).
 *   - Thread safety: entry points may be called from several host threads;
 *     h2o_last_hip_error() is per host thread.
 *   - Calls that overlap on the same cache buffers race; order them on one
 *     stream.
 */
#ifndef H2O_H_
#define H2O_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define H2O_ABI_VERSION 4

/* Status codes. */
enum h2o_status {
  H2O_OK = 0,
  H2O_EINVAL = -1,       /* null / misaligned pointer, bad sizes, n_occ out of range */
  H2O_EUNSUPPORTED = -2, /* valid but not implemented: D not in {64,128}, chunk straddling capacity,
                            sizes past the 32-bit index range (q_g*T or C+T above 2^22,
                            B*Hkv*(C+T) or B*Hq*T*D above 2^31 - 1), ... */
  H2O_EWORKSPACE = -3,   /* ws_bytes smaller than h2o_workspace_bytes() or ws NULL */
  H2O_EHIP = -4          /* a HIP launch failed; see h2o_last_hip_error() */
};

/* Element type of q, k_new, v_new and out, and of a NATIVE cache. */
enum h2o_dtype { H2O_F32 = 0, H2O_BF16 = 1 };

/* Cache buffer format. */
enum h2o_cache_fmt {
  H2O_CACHE_NATIVE = 0, /* k, v: (B,Hkv,C,D) of `dtype` */
  H2O_CACHE_INT8 = 1,   /* k, v: int8 codes (B,Hkv,C,D); k_scale, v_scale: fp16 (B,Hkv,C) */
  H2O_CACHE_INT4 = 2    /* k, v: uint8 (B,Hkv,C,D/2), element 2i in the low nibble of byte i;
                           k_scale, v_scale, k_zero, v_zero: fp16 (B,Hkv,C) */
};

/* Score used to choose the slots to overwrite once the cache is full
 * ("Learning how to Forget", §3.1.1).  The stored scores are the cumulative
 * summed weights per (b, KV head, slot) under every policy; the policy only
 * changes the value the slots are ranked by. */
enum h2o_policy {
  H2O_POLICY_H2O = 0,  /* the cumulative score */
  H2O_POLICY_NORM = 1, /* score / (pos + T - token_pos[slot]): the score averaged over the
                          queries that have attended the slot; needs token_pos */
  H2O_POLICY_ORIG = 2  /* score summed over the batch rows (fp32, b ascending); every batch
                          row selects the same slots */
};

/* Problem sizes.  B batch, Hq query heads, Hkv KV heads (Hq % Hkv == 0),
 * D head dimension (64 or 128), C cache capacity in slots, T chunk length.
 * scale: softmax scale applied to q.k; 0 selects 1/sqrt(D). */
typedef struct {
  int32_t B, Hq, Hkv, D, C, T;
  int32_t dtype;     /* enum h2o_dtype */
  int32_t cache_fmt; /* enum h2o_cache_fmt */
  int32_t policy;    /* enum h2o_policy */
  float scale;
} h2o_dims;

/* One layer's cache state.  Caller-owned device buffers.
 *   k, v        see enum h2o_cache_fmt
 *   k_scale...  fp16 bit patterns (B,Hkv,C); NULL for NATIVE; zeros only for INT4
 *   scores      fp32 (B,Hkv,C): running H2O scores of the occupied slots
 *   token_pos   int32 (B,Hkv,C): absolute token position held by each slot, or NULL
 *               when the caller does not track positions */
typedef struct {
  void *k, *v;
  uint16_t *k_scale, *v_scale;
  uint16_t *k_zero, *v_zero;
  float *scores;
  int32_t *token_pos;
} h2o_cache;

/* Library and error reporting. */
int h2o_abi_version(void);
const char *h2o_status_str(int status);
/* hipError_t of the last failed launch on this host thread (0 if none). */
int h2o_last_hip_error(void);

/* Device workspace needed by h2o_sdpa_scoresum / h2o_evict_topk /
 * h2o_chunk_step for these sizes, in bytes (covers every n_occ <= C).
 * Returns 0 when `d` is invalid. */
size_t h2o_workspace_bytes(const h2o_dims *d);

/* Attention of one chunk with exact summed weights; changes no cache state.
 * ("Learning how to Forget", §A.7: softmax(mask(scale Q K^T)) and the summed
 * weights it names; §A.1: causal mask by token position -- with the chunk
 * attending before it is written, every occupied slot is visible and the
 * chunk's own keys are causal.)
 *   n_occ   occupied slots, 0 <= n_occ <= C; slots 0..n_occ-1 are attended
 *   q       (B,Hq,T,D) dtype          k_new, v_new (B,Hkv,T,D) dtype
 *   out     (B,Hq,T,D) dtype: attention output
 *   wsum    fp32 (B,Hkv,n_occ+T): column j < n_occ is slot j, column n_occ+t is
 *           chunk token t; each is sum over the chunk's queries and the q_g
 *           heads of the group of the softmax weight on that key
 *   lse     fp32 (B,Hq,T) natural-log softmax normaliser, or NULL
 *   ws      workspace of at least h2o_workspace_bytes(d) bytes */
int h2o_sdpa_scoresum(const h2o_dims *d, const h2o_cache *cache, int32_t n_occ,
                      const void *q, const void *k_new, const void *v_new,
                      void *out, float *wsum, float *lse,
                      void *ws, size_t ws_bytes, void *stream);

/* Score update, slot selection and replay log (aimodeling article: H2O score =
 * cumulative attention-weight sums, lowest evicted; "Learning how to Forget",
 * §3.1: left-to-right fill, B*Hkv*T slots per chunk; §3.2: replay log).
 *   scores[j] += wsum[j] for j < n_occ.
 *   If n_occ + T <= C: slot_log[b,g,t] = n_occ + t.
 *   If n_occ == C:     slot_log[b,g,:] = the T slots with the smallest ranking
 *                      value (enum h2o_policy) under (value, slot index), in
 *                      ascending slot order.
 *   Then for each t: scores[slot_log[t]] = wsum[n_occ+t] and, if token_pos is
 *   not NULL, token_pos[slot_log[t]] = pos + t.  K/V buffers are not touched.
 *   n_occ < C < n_occ + T, or T > C when n_occ == C, returns H2O_EUNSUPPORTED;
 *   H2O_POLICY_NORM without token_pos returns H2O_EINVAL.
 *   C must be <= 65536.
 *   slot_log: int32 (B,Hkv,T).
 *   ws: optional scratch (may be NULL; otherwise 16-byte aligned).  With at
 *   least h2o_workspace_bytes(d) bytes, short chunks (T up to about
 *   C / (2 * ceil(C / 1024))) select over many workgroups per head; the
 *   selected slots are the same either way. */
int h2o_evict_topk(const h2o_dims *d, h2o_cache *cache, int32_t n_occ, int64_t pos,
                   const float *wsum, int32_t *slot_log,
                   void *ws, size_t ws_bytes, void *stream);

/* Write the chunk's keys and values into the slots of slot_log, unchanged
 * ("Learning how to Forget", §A.8: scatter along the slot axis with the head
 * dimension contiguous).  NATIVE caches only (H2O_EINVAL otherwise).  Rows
 * whose slot_log entry lies outside [0, C) are skipped. */
int kv_scatter(const h2o_dims *d, h2o_cache *cache, const void *k_new, const void *v_new,
               const int32_t *slot_log, void *stream);

/* Quantise the chunk's keys and values per row and write codes, scales (and
 * zero points) into the slots of slot_log.  INT8 or INT4 caches only
 * (H2O_EINVAL for NATIVE).  The aimodeling.com article on the KeysAndValues
 * release names 8-bit and 4-bit cache buffers (4-bit: a quarter of the cache
 * memory), and "Learning how to Forget" §2 lists quantised caches among the
 * library's buffers; neither gives a scheme.  This library uses, per slot
 * and KV head, with IEEE fp32 operations:
 *   INT8: a = max|x|; s = fp16(a/127); c = clamp(rne(x/s), -127, 127)
 *   INT4: z = fp16(min x); s = fp16((max x - min x)/15);
 *         c = clamp(rne((x - z)/s), 0, 15)
 *   with all codes 0 when s == 0.  Dequantised value: c*s (+ z).  Rows whose
 *   slot_log entry lies outside [0, C) are skipped. */
int kv_quant_pack(const h2o_dims *d, h2o_cache *cache, const void *k_new, const void *v_new,
                  const int32_t *slot_log, void *stream);

/* Inspection helper: dequantise (or widen) the first n_slots slots of every
 * (b, g) of the cache into fp32 k_out, v_out of shape (B,Hkv,n_slots,D). */
int kv_dequant_unpack(const h2o_dims *d, const h2o_cache *cache, int32_t n_slots,
                      float *k_out, float *v_out, void *stream);

/* The whole chunk step ("Learning how to Forget", §3.1: a chunk of T tokens
 * attends to the cache plus itself, and B*Hkv*T slots are then overwritten
 * by its keys and values; §3.1.1: the H2O score of a slot is its cumulative
 * summed attention weight; §3.2: the decisions go to a replay log):
 * h2o_sdpa_scoresum, then h2o_evict_topk, then kv_scatter (NATIVE) or
 * kv_quant_pack (INT8/INT4), enqueued on `stream`.  For short chunks the
 * kernels are merged with the same results: the selection's first kernel
 * forms the summed weights from the logits the attention stored, and its
 * last kernel writes the rows.  wsum may be NULL (the sums then live in the
 * workspace).  After the call the caller's occupancy
 * is min(n_occ + T, C) and its position pos + T. */
int h2o_chunk_step(const h2o_dims *d, h2o_cache *cache, int32_t n_occ, int64_t pos,
                   const void *q, const void *k_new, const void *v_new,
                   void *out, float *wsum, int32_t *slot_log,
                   void *ws, size_t ws_bytes, void *stream);

/* h2o_chunk_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same work, with the workspace taken from a device-resident array of
 * H2O_NOALLOC_SCRATCH_BYTES that the library reserves on each GPU it runs on
 * and holds until the process ends.  The call allocates and frees nothing.
 *   Arguments, results and return codes are those of h2o_chunk_step without
 *   ws / ws_bytes; wsum may be NULL (the sums then live in the array).
 *   H2O_EWORKSPACE: the workspace this call needs (row normalisers, key-split
 *   partials, stored logits, and the sums when wsum is NULL) exceeds
 *   H2O_NOALLOC_SCRATCH_BYTES.  The array is per GPU: `stream` must belong to
 *   the current device.  Every call on a GPU uses that GPU's one array, and
 *   no kernel reads a byte of it the same call has not written, so it is
 *   never cleared; calls that overlap in time on one GPU (several streams,
 *   or host threads without ordering) race on it. */
#define H2O_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int h2o_chunk_step_noalloc(const h2o_dims *d, h2o_cache *cache, int32_t n_occ, int64_t pos,
                           const void *q, const void *k_new, const void *v_new, void *out,
                           float *wsum, int32_t *slot_log, void *stream);

/* Replay step ("Learning how to Forget", §3.2: replay caches act like normal
 * KV caches except that eviction decisions are replayed from the log): the
 * attention of h2o_sdpa_scoresum without the summed weights (no scoring, no
 * selection), then the chunk's keys and values are written (quantised for
 * INT8/INT4) into the slots of a logged decision, and token_pos (if not NULL)
 * is set to pos + t for slot_log[b,g,t].  Scores are left untouched.
 *   slot_log  int32 (B,Hkv,T): a row of the replay log, e.g. as written by
 *             h2o_evict_topk / h2o_chunk_step for the same step; entries
 *             outside [0, C) are skipped.
 *   out       (B,Hq,T,D) dtype.  ws: at least h2o_workspace_bytes(d) bytes.
 *   n_occ, pos and the return codes are as for h2o_chunk_step; after the call
 *   the caller's occupancy is min(n_occ + T, C) and its position pos + T. */
int h2o_replay_step(const h2o_dims *d, h2o_cache *cache, int32_t n_occ, int64_t pos,
                    const void *q, const void *k_new, const void *v_new, void *out,
                    const int32_t *slot_log, void *ws, size_t ws_bytes, void *stream);

/* Gradients of the chunk attention ("Learning how to Forget", §3.2: the
 * fine-tuning pass differentiates each chunk's SDPA call by reverse mode;
 * §A.10: the attention interface with summed weights has a backward).  For
 * the attention of h2o_sdpa_scoresum with the same d, cache, n_occ and chunk,
 * and an upstream gradient dout = dL/d(out):
 *   dq = scale dS K,  dk = scale dS^T Q,  dv = P^T dout,
 *   dS = P o (dP - rowsum(P o dP)),  dP = dout V^T,
 * with P the masked softmax (cache slots visible, chunk keys causal) and the
 * keys K, V = the n_occ cache rows followed by the chunk's.  dk and dv of a KV
 * head are summed over its q_g query heads.  The summed weights carry no
 * gradient.  P is recomputed from lse; the row term rowsum(P o dP) (which
 * equals rowsum(dout o out)) is summed in fp32 from the recomputed P and dP,
 * so the forward's output is not needed.  P and dS enter the products as
 * bf16, all sums are fp32.
 *   q, k_new, v_new, cache   as for h2o_sdpa_scoresum (read only)
 *   lse    (B,Hq,T) fp32: the forward's natural-log row normalisers (the lse
 *          output of h2o_sdpa_scoresum)
 *   dout   (B,Hq,T,D) bf16
 *   dq     (B,Hq,T,D) fp32, written
 *   dk_cache, dv_cache  (B,Hkv,C,D) fp32: rows < n_occ written, the rest
 *          untouched (may be NULL when n_occ == 0)
 *   dk_new, dv_new      (B,Hkv,T,D) fp32, written
 *   ws     at least h2o_workspace_bytes(d) bytes (16-byte aligned)
 * Supported: dtype H2O_BF16, cache_fmt H2O_CACHE_NATIVE, D = 128; otherwise
 * H2O_EUNSUPPORTED.  Null or misaligned buffers: H2O_EINVAL.  Deterministic
 * (no atomics). */
int h2o_sdpa_backward(const h2o_dims *d, const h2o_cache *cache, int32_t n_occ,
                      const void *q, const void *k_new, const void *v_new,
                      const float *lse, const void *dout,
                      float *dq, float *dk_cache, float *dv_cache, float *dk_new, float *dv_new,
                      void *ws, size_t ws_bytes, void *stream);

/* Kernel timing, for measurement.  While enabled, every kernel the library
 * launches is bracketed by two hipEvents recorded on the caller's stream (the
 * events come from a pool the library owns; no device memory is allocated).
 * h2o_profile_read waits for the recorded events, adds their elapsed times to
 * per-kind totals and copies the totals (milliseconds) and launch counts into
 * arrays of at least H2O_K_COUNT entries (H2O_EINVAL otherwise). */
enum h2o_kernel_kind {
  H2O_K_ATTN_A = 0,   /* attention output and row normalisers */
  H2O_K_ATTN_B = 1,   /* summed weights */
  H2O_K_EVICT = 2,    /* score update, selection, replay log */
  H2O_K_KV_WRITE = 3, /* slot overwrite / quantise */
  H2O_K_ATTN_COMBINE = 4, /* merge of key-split partial outputs (small chunks) */
  H2O_K_BWD_ROWS = 5, /* backward: row terms rowsum(P o dP) and log2 normalisers */
  H2O_K_BWD_DQ = 6,   /* backward: dq */
  H2O_K_BWD_DKDV = 7, /* backward: dk, dv */
  H2O_K_COUNT = 8
};
int h2o_profile_enable(int on);
int h2o_profile_read(double *total_ms, int64_t *launches, int n);
int h2o_profile_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* H2O_H_ */
