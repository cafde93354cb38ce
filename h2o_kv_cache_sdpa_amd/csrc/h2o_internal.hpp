// Internal launch interface of libh2o.so (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/h2o.h"

// Device-side index checks of the debug build (H2O_DEBUG): a failed check
// ends the kernel with a trap, so a write that would land outside its
// buffer becomes a launch error instead of silent corruption.  The release
// build compiles them away.
#ifdef H2O_DEBUG
#define H2O_DEVICE_CHECK(cond) \
  do {                         \
    if (!(cond)) __builtin_trap(); \
  } while (0)
#else
#define H2O_DEVICE_CHECK(cond) ((void)0)
#endif

namespace h2o {

enum : int { DT_F32 = 0, DT_BF16 = 1 };
enum : int { FMT_NATIVE = 0, FMT_INT8 = 1, FMT_INT4 = 2 };

// Everything the attention passes read or write.  Shapes (row-major):
//   q (B,Hq,T,D)  kn, vn (B,Hkv,T,D)  kc, vc cache (B,Hkv,C,D) or codes
//   out (B,Hq,T,D)  wsum (B,Hkv,n_occ+T)  lse2 (B,Hq,T) log2-domain normaliser
struct AttnArgs {
  const void *q, *kn, *vn;
  const void *kc, *vc;
  const uint16_t *ks, *vs, *kz, *vz;  // fp16 scale / zero bit patterns (B,Hkv,C)
  void *out;
  float *wsum;     // null: output only (pass B is skipped)
  float *lse2;     // workspace: m + log2(l) with logits measured in units of log2
  float *lse_nat;  // optional natural-log copy for the caller (may be null)
  // Key-split pass A (nsplit > 1): split s of row r leaves its unnormalised
  // output in part[(s*B*Hq*T + r)*D ..] and (m, l) in part_ml[2*(s*B*Hq*T + r)];
  // a combine kernel merges them into out and lse2.
  float *part, *part_ml;
  int nsplit;
  // Short chunks (bf16, D = 128, qg*T <= LOGIT_ROWS_MAX): pass A also stores
  // each row's logits q.k (after the cache's scale / zero) at
  // lg[(grp*qg*T + r)*lg_stride + j], and the summed weights come from them
  // instead of a second pass over K.  Null otherwise.
  float *lg;
  int lg_stride;
  // With lg set, defer_b leaves the summed weights (and the merge of the key
  // splits) to the selection's first kernel, which forms them from the
  // stored logits (launch_evict with these arguments).
  int defer_b;
  int B, Hq, Hkv, D, C, T, qg, n_occ;
  int dtype, cache_fmt;
  float sl2;  // softmax scale * log2(e)
};

struct EvictArgs {
  float *scores;        // (B,Hkv,C)
  int32_t *token_pos;   // (B,Hkv,C); may be null for the h2o and h2o_orig policies
  const float *wsum;    // (B,Hkv,n_occ+T)
  int32_t *slot_log;    // (B,Hkv,T)
  int groups, C, T, n_occ;
  int B, Hkv, policy;   // groups = B * Hkv; policy: enum h2o_policy
  long long pos;
};

struct KvWriteArgs {
  void *kc, *vc;
  uint16_t *ks, *vs, *kz, *vz;
  const void *kn, *vn;
  const int32_t *slot_log;
  int32_t *token_pos;  // when set, token_pos[slot_log[t]] = pos + t (replay)
  long long pos;
  int groups, C, T, D;
  int dtype, cache_fmt;
};

// Backward of the chunk attention (bf16, native cache, D = 128).
struct BwdArgs {
  const void *q, *kn, *vn, *kc, *vc, *dout;
  const float *lse;  // (B,Hq,T) natural-log row normalisers of the forward
  float *l2, *dd;    // workspace (B,Hq,T): lse * log2(e), sum_j P_rj dP_rj
  float *dq;         // (B,Hq,T,D)
  float *dkc, *dvc;  // (B,Hkv,C,D), rows < n_occ
  float *dkn, *dvn;  // (B,Hkv,T,D)
  int B, Hq, Hkv, C, T, qg, n_occ;
  float scale, sl2;
};
hipError_t launch_bwd_dq(const BwdArgs &a, hipStream_t s);  // row terms, then dQ (attn_bwd_dq.hip)
hipError_t launch_attn_backward(const BwdArgs &a, hipStream_t s);

// Brackets one kernel launch with hipEvents on `s` while timing is enabled
// (h2o_profile_enable); kind is an enum h2o_kernel_kind value.
class KernelTimer {
 public:
  KernelTimer(int kind, hipStream_t s);
  ~KernelTimer();
  KernelTimer(const KernelTimer &) = delete;
  KernelTimer &operator=(const KernelTimer &) = delete;

 private:
  int kind_;
  hipStream_t stream_;
  hipEvent_t start_ = nullptr;
};

hipError_t launch_attn_simple(const AttnArgs &a, hipStream_t s);
hipError_t launch_attn_mfma(const AttnArgs &a, hipStream_t s);
hipError_t launch_attn_native_d128(const AttnArgs &a, hipStream_t s);
constexpr int LOGIT_ROWS_MAX = 16;
// Pass B (summed weights) for bf16 queries, D = 128, any cache format.
hipError_t launch_attn_b_native(const AttnArgs &a, hipStream_t s);
// Summed weights from the logits pass A stored (a.lg).
hipError_t launch_attn_b_logits(const AttnArgs &a, hipStream_t s);
// Pass A alone for int8 / int4 caches, bf16, D = 128.
hipError_t launch_attn_a_quant_d128(const AttnArgs &a, hipStream_t s);
// Pass A alone for short chunks (qg * T <= 16), bf16 queries, D = 128, every
// cache format; the caller brackets it with its kernel timer.
hipError_t launch_attn_a_short_d128(const AttnArgs &a, hipStream_t s);
// Key splits pass A uses for these sizes (1 unless the row blocks alone
// cannot fill the chip); the workspace must hold attn_split_floats() floats.
int attn_splits(int B, int Hq, int Hkv, int D, int T, int n_occ, int dtype, int cache_fmt);
// Merge of the key-split partials of pass A into out and lse2 (D = 128).
hipError_t launch_attn_combine(const AttnArgs &a, hipStream_t s);
size_t attn_split_floats(int B, int Hq, int D, int T, int nsplit);
// ws / ws_bytes: optional candidate buffer of evict_workspace_bytes() bytes;
// with it, short chunks select over many workgroups per head.
// kv (optional): the chunk's K/V write.  When the selection can do it in the
// same launch (two-pass shape, native cache, short chunk) it does and sets
// *kv_done; otherwise the caller launches launch_kv_write afterwards.
// lg (optional): attention arguments whose stored logits the selection sums
// itself (a.defer_b was set for pass A); requires the two-pass shape
// (evict_two_pass), otherwise hipErrorInvalidValue.
hipError_t launch_evict(const EvictArgs &a, void *ws, size_t ws_bytes, hipStream_t s,
                        const KvWriteArgs *kv = nullptr, bool *kv_done = nullptr,
                        const AttnArgs *lg = nullptr);
size_t evict_workspace_bytes(int groups, int C, int T);
// True when launch_evict takes the two-pass shape (slice candidates + pick).
bool evict_two_pass(const EvictArgs &a, size_t ws_bytes);
hipError_t launch_kv_write(const KvWriteArgs &a, hipStream_t s);
hipError_t launch_dequant(const KvWriteArgs &a, int n_slots, float *kout, float *vout, hipStream_t s);

}  // namespace h2o
