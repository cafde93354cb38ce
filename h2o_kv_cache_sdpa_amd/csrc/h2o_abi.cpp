// C ABI of libh2o.so: host-side validation and dispatch.  Every argument is
// checked before anything is enqueued; no entry point allocates, frees or
// synchronises.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/h2o.h"
#include "h2o_internal.hpp"

// Workspace of h2o_chunk_step_noalloc: one array per GPU, reserved when the
// code object is loaded on that GPU and held until the process ends.  Host
// code never uses this name as a device address: the address comes from
// hipGetSymbolAddress (scratch_address below), once per device.
static __device__ __align__(256) unsigned char scratch[H2O_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local int g_last_hip_error = 0;

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validates sizes and enums.  Returns H2O_OK, H2O_EINVAL or H2O_EUNSUPPORTED.
int check_dims(const h2o_dims *d) {
  if (!d) return H2O_EINVAL;
  if (d->B < 1 || d->Hq < 1 || d->Hkv < 1 || d->C < 1 || d->T < 1 || d->D < 1) return H2O_EINVAL;
  if (d->Hq % d->Hkv != 0) return H2O_EINVAL;
  if (d->dtype != H2O_F32 && d->dtype != H2O_BF16) return H2O_EINVAL;
  if (d->cache_fmt < H2O_CACHE_NATIVE || d->cache_fmt > H2O_CACHE_INT4) return H2O_EINVAL;
  if (!(std::isfinite(d->scale) && d->scale >= 0.f)) return H2O_EINVAL;
  if (d->policy < H2O_POLICY_H2O || d->policy > H2O_POLICY_ORIG) return H2O_EUNSUPPORTED;
  if (d->D != 64 && d->D != 128) return H2O_EUNSUPPORTED;
  // Index arithmetic inside the kernels uses 32-bit integers: byte offsets
  // of up to 2^22 rows of 256 bytes, score / position / sum indices of up to
  // B*Hkv*(C+T) elements, and query-row indices of up to B*Hq*T.
  const int64_t rows = static_cast<int64_t>(d->Hq / d->Hkv) * d->T;
  const int64_t keys = static_cast<int64_t>(d->C) + d->T;
  const int64_t groups = static_cast<int64_t>(d->B) * d->Hkv;
  if (rows > (1 << 22) || keys > (1 << 22)) return H2O_EUNSUPPORTED;
  if (groups * keys > INT32_MAX) return H2O_EUNSUPPORTED;
  if (static_cast<int64_t>(d->B) * d->Hq * d->T * d->D > INT32_MAX) return H2O_EUNSUPPORTED;
  return H2O_OK;
}

// Workspace of the attention passes: two fp32 planes of (B,Hq,T) -- the
// log2-domain row normaliser and, for INT4 caches, the per-row sum of q.
size_t lse_bytes(const h2o_dims *d) {
  return align_up(2 * sizeof(float) * static_cast<size_t>(d->B) * d->Hq * d->T);
}

// Partial outputs of a key-split pass A (zero when the step is not split).
size_t split_bytes(const h2o_dims *d, int n_occ) {
  const int ns = h2o::attn_splits(d->B, d->Hq, d->Hkv, d->D, d->T, n_occ, d->dtype, d->cache_fmt);
  return align_up(sizeof(float) * h2o::attn_split_floats(d->B, d->Hq, d->D, d->T, ns));
}

// Short chunks keep pass A's logits for the summed weights (bf16, D = 128,
// at most LOGIT_ROWS_MAX query rows per KV group); rows padded to 64 keys.
bool use_logits(const h2o_dims *d) {
  return d->dtype == H2O_BF16 && d->D == 128 && (d->Hq / d->Hkv) * d->T <= h2o::LOGIT_ROWS_MAX;
}
int logit_stride(const h2o_dims *d, int n_occ) { return (n_occ + d->T + 63) / 64 * 64; }
size_t logit_bytes(const h2o_dims *d, int n_occ) {
  if (!use_logits(d)) return 0;
  return align_up(sizeof(float) * static_cast<size_t>(d->B) * d->Hq * d->T * logit_stride(d, n_occ));
}

// Everything the attention passes keep in the workspace, in this order.
size_t attn_ws_bytes(const h2o_dims *d, int n_occ) {
  return lse_bytes(d) + split_bytes(d, n_occ) + logit_bytes(d, n_occ);
}

// Candidate lists of the short-chunk slot selection (zero when not used).
size_t evict_bytes(const h2o_dims *d) {
  const int heads = d->B * d->Hkv;
  return align_up(h2o::evict_workspace_bytes(heads, d->C, d->T));
}

size_t wsum_bytes(const h2o_dims *d, int n_occ) {
  return align_up(sizeof(float) * static_cast<size_t>(d->B) * d->Hkv * (n_occ + d->T));
}

int check_cache_buffers(const h2o_dims *d, const h2o_cache *c) {
  if (!c || !c->k || !c->v) return H2O_EINVAL;
  if (!aligned16(c->k) || !aligned16(c->v)) return H2O_EINVAL;
  if (d->cache_fmt != H2O_CACHE_NATIVE) {
    if (!c->k_scale || !c->v_scale) return H2O_EINVAL;
    if (d->cache_fmt == H2O_CACHE_INT4 && (!c->k_zero || !c->v_zero)) return H2O_EINVAL;
  }
  return H2O_OK;
}

float softmax_scale(const h2o_dims *d) {
  return d->scale > 0.f ? d->scale : static_cast<float>(1.0 / std::sqrt(static_cast<double>(d->D)));
}

int from_hip(hipError_t e) {
  if (e == hipSuccess) return H2O_OK;
  g_last_hip_error = static_cast<int>(e);
  return H2O_EHIP;
}

int check_sdpa(const h2o_dims *d, const h2o_cache *cache, int32_t n_occ, const void *q,
               const void *k_new, const void *v_new, const void *out, const float *wsum,
               const float *lse, const void *ws, size_t ws_bytes, bool need_wsum = true) {
  int st = check_dims(d);
  if (st != H2O_OK) return st;
  if (n_occ < 0 || n_occ > d->C) return H2O_EINVAL;
  if (!q || !k_new || !v_new || !out || (need_wsum && !wsum)) return H2O_EINVAL;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out) ||
      (wsum && !aligned16(wsum)) || (lse && !aligned16(lse)))
    return H2O_EINVAL;
  if (n_occ > 0) {
    st = check_cache_buffers(d, cache);
    if (st != H2O_OK) return st;
  }
  if (!ws || !aligned16(ws) || ws_bytes < attn_ws_bytes(d, n_occ)) return H2O_EWORKSPACE;
  return H2O_OK;
}

int check_evict(const h2o_dims *d, const h2o_cache *cache, int32_t n_occ, int64_t pos,
                const float *wsum, const int32_t *slot_log) {
  int st = check_dims(d);
  if (st != H2O_OK) return st;
  if (!cache || !cache->scores || !wsum || !slot_log) return H2O_EINVAL;
  if (n_occ < 0 || n_occ > d->C || pos < 0) return H2O_EINVAL;
  if (cache->token_pos && pos + d->T > INT32_MAX) return H2O_EINVAL;
  if (d->policy == H2O_POLICY_NORM && !cache->token_pos) return H2O_EINVAL;  // ages need positions
  if (!(n_occ + static_cast<int64_t>(d->T) <= d->C || n_occ == d->C)) return H2O_EUNSUPPORTED;
  if (n_occ == d->C && d->T > d->C) return H2O_EUNSUPPORTED;  // cannot evict more than C slots
  if (d->C > 65536) return H2O_EUNSUPPORTED;
  return H2O_OK;
}

int check_write(const h2o_dims *d, const h2o_cache *cache, const void *k_new, const void *v_new,
                const int32_t *slot_log) {
  int st = check_dims(d);
  if (st != H2O_OK) return st;
  if (!k_new || !v_new || !slot_log || !aligned16(k_new) || !aligned16(v_new)) return H2O_EINVAL;
  return check_cache_buffers(d, cache);
}

h2o::AttnArgs attn_args(const h2o_dims *d, const h2o_cache *cache, int32_t n_occ, const void *q,
                        const void *k_new, const void *v_new, void *out, float *wsum, float *lse,
                        void *ws) {
  h2o::AttnArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = q;
  a.kn = k_new;
  a.vn = v_new;
  if (cache) {
    a.kc = cache->k;
    a.vc = cache->v;
    a.ks = cache->k_scale;
    a.vs = cache->v_scale;
    a.kz = cache->k_zero;
    a.vz = cache->v_zero;
  }
  a.out = out;
  a.wsum = wsum;
  a.lse2 = static_cast<float *>(ws);
  a.lse_nat = lse;
  a.nsplit = h2o::attn_splits(d->B, d->Hq, d->Hkv, d->D, d->T, n_occ, d->dtype, d->cache_fmt);
  a.part = reinterpret_cast<float *>(static_cast<char *>(ws) + lse_bytes(d));
  a.part_ml = a.part + static_cast<size_t>(a.nsplit) * d->B * d->Hq * d->T * d->D;
  if (wsum && use_logits(d)) {
    a.lg = reinterpret_cast<float *>(static_cast<char *>(ws) + lse_bytes(d) + split_bytes(d, n_occ));
    a.lg_stride = logit_stride(d, n_occ);
  }
  a.B = d->B;
  a.Hq = d->Hq;
  a.Hkv = d->Hkv;
  a.D = d->D;
  a.C = d->C;
  a.T = d->T;
  a.qg = d->Hq / d->Hkv;
  a.n_occ = n_occ;
  a.dtype = d->dtype;
  a.cache_fmt = d->cache_fmt;
  a.sl2 = static_cast<float>(static_cast<double>(softmax_scale(d)) * 1.4426950408889634074);
  return a;
}

int launch_sdpa(const h2o::AttnArgs &a, hipStream_t s) {
  if (a.dtype == h2o::DT_BF16) return from_hip(h2o::launch_attn_mfma(a, s));
  return from_hip(h2o::launch_attn_simple(a, s));
}

h2o::KvWriteArgs write_args(const h2o_dims *d, h2o_cache *cache, const void *k_new,
                            const void *v_new, const int32_t *slot_log) {
  h2o::KvWriteArgs w;
  std::memset(&w, 0, sizeof(w));
  w.kc = cache->k;
  w.vc = cache->v;
  w.ks = cache->k_scale;
  w.vs = cache->v_scale;
  w.kz = cache->k_zero;
  w.vz = cache->v_zero;
  w.kn = k_new;
  w.vn = v_new;
  w.slot_log = slot_log;
  w.groups = d->B * d->Hkv;
  w.C = d->C;
  w.T = d->T;
  w.D = d->D;
  w.dtype = d->dtype;
  w.cache_fmt = d->cache_fmt;
  w.token_pos = nullptr;
  w.pos = 0;
  return w;
}

h2o::EvictArgs evict_args(const h2o_dims *d, h2o_cache *cache, int32_t n_occ, int64_t pos,
                          const float *wsum, int32_t *slot_log) {
  h2o::EvictArgs e;
  e.scores = cache->scores;
  e.token_pos = cache->token_pos;
  e.wsum = wsum;
  e.slot_log = slot_log;
  e.groups = d->B * d->Hkv;
  e.B = d->B;
  e.Hkv = d->Hkv;
  e.policy = d->policy;
  e.C = d->C;
  e.T = d->T;
  e.n_occ = n_occ;
  e.pos = pos;
  return e;
}

}  // namespace

extern "C" {

int h2o_abi_version(void) { return H2O_ABI_VERSION; }

const char *h2o_status_str(int status) {
  switch (status) {
    case H2O_OK: return "ok";
    case H2O_EINVAL: return "invalid argument";
    case H2O_EUNSUPPORTED: return "unsupported configuration";
    case H2O_EWORKSPACE: return "workspace missing or too small";
    case H2O_EHIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int h2o_last_hip_error(void) { return g_last_hip_error; }

size_t h2o_workspace_bytes(const h2o_dims *d) {
  if (check_dims(d) != H2O_OK) return 0;
  return attn_ws_bytes(d, d->C) + wsum_bytes(d, d->C) + evict_bytes(d);
}

int h2o_sdpa_scoresum(const h2o_dims *d, const h2o_cache *cache, int32_t n_occ, const void *q,
                      const void *k_new, const void *v_new, void *out, float *wsum, float *lse,
                      void *ws, size_t ws_bytes, void *stream) {
  const int st = check_sdpa(d, cache, n_occ, q, k_new, v_new, out, wsum, lse, ws, ws_bytes);
  if (st != H2O_OK) return st;
  const h2o::AttnArgs a = attn_args(d, cache, n_occ, q, k_new, v_new, out, wsum, lse, ws);
  return launch_sdpa(a, static_cast<hipStream_t>(stream));
}

int h2o_evict_topk(const h2o_dims *d, h2o_cache *cache, int32_t n_occ, int64_t pos,
                   const float *wsum, int32_t *slot_log, void *ws, size_t ws_bytes,
                   void *stream) {
  const int st = check_evict(d, cache, n_occ, pos, wsum, slot_log);
  if (st != H2O_OK) return st;
  if (ws && !aligned16(ws)) return H2O_EWORKSPACE;
  return from_hip(h2o::launch_evict(evict_args(d, cache, n_occ, pos, wsum, slot_log), ws,
                                    ws ? ws_bytes : 0, static_cast<hipStream_t>(stream)));
}

int h2o_sdpa_backward(const h2o_dims *d, const h2o_cache *cache, int32_t n_occ, const void *q,
                      const void *k_new, const void *v_new, const float *lse, const void *dout,
                      float *dq, float *dk_cache, float *dv_cache, float *dk_new, float *dv_new,
                      void *ws, size_t ws_bytes, void *stream) {
  int st = check_dims(d);
  if (st != H2O_OK) return st;
  if (d->dtype != H2O_BF16 || d->cache_fmt != H2O_CACHE_NATIVE || d->D != 128) return H2O_EUNSUPPORTED;
  if (n_occ < 0 || n_occ > d->C) return H2O_EINVAL;
  const void *need[] = {q, k_new, v_new, lse, dout, dq, dk_new, dv_new};
  for (const void *p : need)
    if (!p || !aligned16(p)) return H2O_EINVAL;
  if (n_occ > 0) {
    if (!dk_cache || !dv_cache || !aligned16(dk_cache) || !aligned16(dv_cache)) return H2O_EINVAL;
    st = check_cache_buffers(d, cache);
    if (st != H2O_OK) return st;
  }
  if (!ws || !aligned16(ws) || ws_bytes < lse_bytes(d)) return H2O_EWORKSPACE;
  h2o::BwdArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = q;
  a.kn = k_new;
  a.vn = v_new;
  if (cache) {
    a.kc = cache->k;
    a.vc = cache->v;
  }
  a.dout = dout;
  a.lse = lse;
  const size_t rows = static_cast<size_t>(d->B) * d->Hq * d->T;
  a.l2 = static_cast<float *>(ws);
  a.dd = a.l2 + rows;
  a.dq = dq;
  a.dkc = dk_cache;
  a.dvc = dv_cache;
  a.dkn = dk_new;
  a.dvn = dv_new;
  a.B = d->B;
  a.Hq = d->Hq;
  a.Hkv = d->Hkv;
  a.C = d->C;
  a.T = d->T;
  a.qg = d->Hq / d->Hkv;
  a.n_occ = n_occ;
  a.scale = softmax_scale(d);
  a.sl2 = static_cast<float>(static_cast<double>(a.scale) * 1.4426950408889634074);
  return from_hip(h2o::launch_attn_backward(a, static_cast<hipStream_t>(stream)));
}

int kv_scatter(const h2o_dims *d, h2o_cache *cache, const void *k_new, const void *v_new,
               const int32_t *slot_log, void *stream) {
  const int st = check_write(d, cache, k_new, v_new, slot_log);
  if (st != H2O_OK) return st;
  if (d->cache_fmt != H2O_CACHE_NATIVE) return H2O_EINVAL;
  return from_hip(h2o::launch_kv_write(write_args(d, cache, k_new, v_new, slot_log),
                                       static_cast<hipStream_t>(stream)));
}

int kv_quant_pack(const h2o_dims *d, h2o_cache *cache, const void *k_new, const void *v_new,
                  const int32_t *slot_log, void *stream) {
  const int st = check_write(d, cache, k_new, v_new, slot_log);
  if (st != H2O_OK) return st;
  if (d->cache_fmt == H2O_CACHE_NATIVE) return H2O_EINVAL;
  return from_hip(h2o::launch_kv_write(write_args(d, cache, k_new, v_new, slot_log),
                                       static_cast<hipStream_t>(stream)));
}

int kv_dequant_unpack(const h2o_dims *d, const h2o_cache *cache, int32_t n_slots, float *k_out,
                      float *v_out, void *stream) {
  int st = check_dims(d);
  if (st != H2O_OK) return st;
  if (n_slots < 1 || n_slots > d->C || !k_out || !v_out) return H2O_EINVAL;
  st = check_cache_buffers(d, cache);
  if (st != H2O_OK) return st;
  h2o::KvWriteArgs w = write_args(d, const_cast<h2o_cache *>(cache), nullptr, nullptr, nullptr);
  return from_hip(h2o::launch_dequant(w, n_slots, k_out, v_out, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

int chunk_step(const h2o_dims *d, h2o_cache *cache, int32_t n_occ, int64_t pos, const void *q,
               const void *k_new, const void *v_new, void *out, float *wsum, int32_t *slot_log, void *ws,
               size_t ws_bytes, void *stream) {
  int st = check_dims(d);
  if (st != H2O_OK) return st;
  if (n_occ < 0 || n_occ > d->C) return H2O_EINVAL;
  const size_t need = attn_ws_bytes(d, n_occ) + (wsum ? 0 : wsum_bytes(d, n_occ));
  if (!ws || !aligned16(ws) || ws_bytes < need) return H2O_EWORKSPACE;
  float *w = wsum ? wsum : reinterpret_cast<float *>(static_cast<char *>(ws) + attn_ws_bytes(d, n_occ));
  st = check_sdpa(d, cache, n_occ, q, k_new, v_new, out, w, nullptr, ws, ws_bytes);
  if (st != H2O_OK) return st;
  st = check_evict(d, cache, n_occ, pos, w, slot_log);
  if (st != H2O_OK) return st;
  st = check_write(d, cache, k_new, v_new, slot_log);
  if (st != H2O_OK) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  // the rest of the workspace, if any, holds the selection's candidate lists
  const size_t used = need;
  const h2o::EvictArgs ea = evict_args(d, cache, n_occ, pos, w, slot_log);
  h2o::AttnArgs aa = attn_args(d, cache, n_occ, q, k_new, v_new, out, w, nullptr, ws);
  // short chunks whose logits pass A stores: when the selection takes the
  // candidate shape, its first kernel forms the summed weights (and merges
  // the key splits) instead of a launch of its own
  aa.defer_b = aa.lg && h2o::evict_two_pass(ea, ws_bytes - used);
  st = launch_sdpa(aa, s);
  if (st != H2O_OK) return st;
  const h2o::KvWriteArgs kv = write_args(d, cache, k_new, v_new, slot_log);
  bool kv_done = false;
  st = from_hip(h2o::launch_evict(ea, static_cast<char *>(ws) + used, ws_bytes - used, s, &kv, &kv_done,
                                  aa.defer_b ? &aa : nullptr));
  if (st != H2O_OK || kv_done) return st;
  return from_hip(h2o::launch_kv_write(kv, s));
}

// Device address of `scratch` on the current device, looked up on the first
// call per device and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices] = {};

int scratch_address(void **addr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return from_hip(e);
  if (dev < 0 || dev >= kMaxDevices) return H2O_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return from_hip(e);
    if (!p) return H2O_EHIP;
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return H2O_OK;
}

}  // namespace

extern "C" {

int h2o_chunk_step(const h2o_dims *d, h2o_cache *cache, int32_t n_occ, int64_t pos, const void *q,
                   const void *k_new, const void *v_new, void *out, float *wsum,
                   int32_t *slot_log, void *ws, size_t ws_bytes, void *stream) {
  return chunk_step(d, cache, n_occ, pos, q, k_new, v_new, out, wsum, slot_log, ws, ws_bytes, stream);
}

int h2o_chunk_step_noalloc(const h2o_dims *d, h2o_cache *cache, int32_t n_occ, int64_t pos,
                           const void *q, const void *k_new, const void *v_new, void *out,
                           float *wsum, int32_t *slot_log, void *stream) {
  int st = check_dims(d);
  if (st != H2O_OK) return st;
  if (n_occ < 0 || n_occ > d->C) return H2O_EINVAL;
  const size_t need = attn_ws_bytes(d, n_occ) + (wsum ? 0 : wsum_bytes(d, n_occ));
  if (need > H2O_NOALLOC_SCRATCH_BYTES) return H2O_EWORKSPACE;
  void *ws = nullptr;
  st = scratch_address(&ws);
  if (st != H2O_OK) return st;
  return chunk_step(d, cache, n_occ, pos, q, k_new, v_new, out, wsum, slot_log, ws,
                    H2O_NOALLOC_SCRATCH_BYTES, stream);
}

int h2o_replay_step(const h2o_dims *d, h2o_cache *cache, int32_t n_occ, int64_t pos, const void *q,
                    const void *k_new, const void *v_new, void *out, const int32_t *slot_log, void *ws,
                    size_t ws_bytes, void *stream) {
  int st = check_sdpa(d, cache, n_occ, q, k_new, v_new, out, nullptr, nullptr, ws, ws_bytes, false);
  if (st != H2O_OK) return st;
  if (!(n_occ + static_cast<int64_t>(d->T) <= d->C || n_occ == d->C)) return H2O_EUNSUPPORTED;
  if (pos < 0 || (cache && cache->token_pos && pos + d->T > INT32_MAX)) return H2O_EINVAL;
  st = check_write(d, cache, k_new, v_new, slot_log);
  if (st != H2O_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = launch_sdpa(attn_args(d, cache, n_occ, q, k_new, v_new, out, nullptr, nullptr, ws), s);
  if (st != H2O_OK) return st;
  h2o::KvWriteArgs w = write_args(d, cache, k_new, v_new, slot_log);
  w.token_pos = cache->token_pos;
  w.pos = pos;
  return from_hip(h2o::launch_kv_write(w, s));
}

}  // extern "C"
