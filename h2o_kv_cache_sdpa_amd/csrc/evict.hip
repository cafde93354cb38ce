// Score accumulate + slot selection + replay log + seeding.
//
// H2O score = cumulative sum of attention weights; the lowest-scoring slots are
// overwritten (aimodeling article on KeysAndValues; "Learning how to Forget",
// §3.1.1).  While the cache has room it fills left to right (§3.1).  Every
// decision goes to the replay log (§3.2).  Ranking key per policy (§3.1.1):
//   h2o       the updated score;
//   h2o_norm  the updated score / (t - t(b,h,j)), t = pos + T (the number of
//             queries that have attended the slot), in IEEE fp32;
//   h2o_orig  the updated scores summed over b (fp32, b ascending); every
//             batch row then takes the same slots.
// The stored scores stay cumulative and per (b, h, slot) under all three.
//
// Selection of the T smallest keys under (score, slot index) is an MSB-first
// radix select over the order-preserving uint32 image of the fp32 ranking
// values (up to 4 passes of 8 bits over the occupied key range, LDS
// histograms), then an index-ordered compaction: a slot is taken if its key is
// below the threshold key, or equal to it and among the first k such slots.
// The replay log row comes out in ascending slot order; chunk token t goes to
// the t-th entry.
//
// Two launch shapes:
//  * one 1024-thread workgroup per (b, KV head) -- per KV head for h2o_orig --
//    that updates, selects and writes (filling, long chunks, no workspace);
//  * for short chunks a candidate pass over slices of SLICE slots (many
//    workgroups per head: update, rank, and keep each slice's T smallest in
//    slot order), then one workgroup per head that selects the T smallest of
//    the candidates.  A slot among the T smallest of its head is among the T
//    smallest of its slice, so both shapes select the same slots.

#include "device_util.hpp"
#include "h2o_internal.hpp"
#include "kv_quant.hpp"
#include "split_merge.hpp"

namespace h2o {
namespace {

constexpr int NT = 1024;     // threads of the per-head workgroups
constexpr int SLICE = 1024;  // slots per candidate workgroup
constexpr int NT_C = 256;    // threads of the candidate workgroups (4 slots each)
constexpr int KV_FUSE_T = 64;  // chunks up to this length: the pick writes the K/V rows
constexpr int QKV_FUSE_T = 4;  // 8/4-bit caches: the pick quantises the rows of chunks up to this length

__device__ __forceinline__ uint32_t ordered_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0 ranks with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int SMALL_T = 8;  // up to this many slots: T rounds of a block minimum (radix select beyond)

struct SelShared {
  uint32_t hist[256];
  uint32_t sel, k;
  uint32_t a[16], b[16];
  uint64_t m64[16];                 // one entry per wavefront (up to 16)
  uint64_t lst[16 * SMALL_T];       // each wavefront's SMALL_T smallest
  uint64_t win[SMALL_T];            // the block's SMALL_T smallest, ascending
};

// Block-wide exclusive scan of two counters; returns the prefixes for this thread.
template <int NTH>
__device__ __forceinline__ void block_scan2(uint32_t a, uint32_t b, uint32_t &ea, uint32_t &eb,
                                            SelShared &sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t ia = a, ib = b;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t na = __shfl_up(ia, o), nb = __shfl_up(ib, o);
    if (lane >= o) {
      ia += na;
      ib += nb;
    }
  }
  if (lane == 63) {
    sh.a[wave] = ia;
    sh.b[wave] = ib;
  }
  __syncthreads();
  uint32_t pa = 0, pb = 0;
  for (int w = 0; w < wave; ++w) {
    pa += sh.a[w];
    pb += sh.b[w];
  }
  ea = pa + ia - a;
  eb = pb + ib - b;
  __syncthreads();  // sh.a / sh.b are free again
}

// Threshold of the `need` smallest of the block's keys; key[k] is valid for
// k < nvalid.  Keys are rewritten relative to the block minimum, so that the
// first digit is taken from the top of the occupied range (the raw top byte --
// sign and exponent -- takes few values).  theta is the (relative) key of the
// need-th smallest; take_eq says how many keys equal to theta are taken.
template <int NTH, int ITEMS>
__device__ __forceinline__ void select_smallest(uint32_t (&key)[ITEMS], int nvalid, uint32_t need,
                                                SelShared &sh, uint32_t &theta, uint32_t &take_eq) {
  constexpr int NW = NTH / 64;
  const int tid = threadIdx.x, lane = tid & 63;
  {
    uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
      if (k < nvalid) {
        kmin = min(kmin, key[k]);
        kmax = max(kmax, key[k]);
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      kmin = min(kmin, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmin), o)));
      kmax = max(kmax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmax), o)));
    }
    if (lane == 0) {
      sh.a[tid >> 6] = kmin;
      sh.b[tid >> 6] = kmax;
    }
    __syncthreads();
    kmin = sh.a[0];
    kmax = sh.b[0];
    for (int wv = 1; wv < NW; ++wv) {
      kmin = min(kmin, sh.a[wv]);
      kmax = max(kmax, sh.b[wv]);
    }
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) key[k] -= kmin;  // invalid keys are never counted
    const uint32_t range = kmax - kmin;
    __syncthreads();
    if (tid == 0) sh.k = range ? 32 - __builtin_clz(range) : 0;  // significant bits of the range
  }
  __syncthreads();
  const int nbits = static_cast<int>(sh.k);
  __syncthreads();
  const int npass = (nbits + 7) / 8;

  uint32_t prefix = 0, pmask = 0;
  for (int pass = 0; pass < npass; ++pass) {
    // digit p covers bits [shift, shift + width) counted from the top of the range
    int shift = nbits - 8 * (pass + 1), width = 8;
    if (shift < 0) {
      width += shift;
      shift = 0;
    }
    const uint32_t dmask = (1u << width) - 1u;
    for (int e = tid; e < 256; e += NTH) sh.hist[e] = 0;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {  // one LDS atomic per key
      if (k < nvalid && (key[k] & pmask) == prefix) atomicAdd(&sh.hist[(key[k] >> shift) & dmask], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      const uint32_t c0 = sh.hist[4 * tid], c1 = sh.hist[4 * tid + 1];
      const uint32_t c2 = sh.hist[4 * tid + 2], c3 = sh.hist[4 * tid + 3];
      const uint32_t s = c0 + c1 + c2 + c3;
      uint32_t inc = s;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t n = __shfl_up(inc, o);
        if (tid >= o) inc += n;
      }
      const uint32_t excl = inc - s;
      if (excl < need && need <= inc) {
        uint32_t c = excl;
        uint32_t d = 4u * tid;
        if (c + c0 < need) {
          c += c0;
          ++d;
          if (c + c1 < need) {
            c += c1;
            ++d;
            if (c + c2 < need) {
              c += c2;
              ++d;
            }
          }
        }
        sh.sel = d;
        sh.k = need - c;
        const uint32_t dd = d - 4u * tid;
        sh.b[0] = dd == 0 ? c0 : dd == 1 ? c1 : dd == 2 ? c2 : c3;  // keys in the digit
      }
    }
    __syncthreads();
    prefix |= sh.sel << shift;
    pmask |= dmask << shift;
    need = sh.k;
    // Every key of the boundary digit is taken: the keys below prefix + 2^shift
    // are exactly the selection, no lower digit to resolve (common for
    // distinct scores after two digits).
    const bool whole = shift > 0 && need == sh.b[0] &&
                       static_cast<uint64_t>(prefix) + (1ull << shift) <= 0xffffffffull;
    __syncthreads();
    if (whole) {
      theta = prefix + (1u << shift);
      take_eq = 0;
      return;
    }
  }
  theta = prefix;
  take_eq = need;
}

// Block-wide minimum of (key << 32 | slot): for T = 1 the selection is the
// smallest key, ties to the lowest slot.  Every thread gets the result.
template <int NTH>
__device__ __forceinline__ uint64_t block_min_u64(uint64_t v, uint64_t *sh64) {
  constexpr int NW = NTH / 64;
  v = wave_min_u64(v);
  if constexpr (NW == 1) {
    return v;
  } else {
    const int lane = threadIdx.x & 63;
    if (lane == 0) sh64[threadIdx.x >> 6] = v;
    __syncthreads();
    return wave_min_u64(lane < NW ? sh64[lane] : ~0ull);
  }
}

// The T <= SMALL_T smallest of the block's (key << 32 | slot) values u[k]
// (~0ull: no value), ascending, in sh.win[0 .. T) on return (every thread
// calls; the slice or candidate list holds at least T values).  Each
// wavefront lists its own T smallest (T rounds of the wavefront minimum, no
// barrier between them); wavefront 0 then takes the T smallest of the lists.
// The values are distinct, so a round's minimum leaves exactly one entry.
template <int NTH, int ITEMS>
__device__ __forceinline__ void block_smallest(uint64_t (&u)[ITEMS], int T, SelShared &sh) {
  constexpr int NW = NTH / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int r = 0; r < T; ++r) {
    uint64_t m = u[0];
#pragma unroll
    for (int k = 1; k < ITEMS; ++k) m = u[k] < m ? u[k] : m;
    m = wave_min_u64(m);
    if (lane == 0) (NW == 1 ? sh.win[r] : sh.lst[wave * T + r]) = m;
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) u[k] = u[k] == m ? ~0ull : u[k];
  }
  __syncthreads();
  if (NW > 1 && wave == 0) {
    // NW * T <= 128 listed values: two per lane
    uint64_t c0 = lane < NW * T ? sh.lst[lane] : ~0ull;
    uint64_t c1 = lane + 64 < NW * T ? sh.lst[lane + 64] : ~0ull;
    for (int r = 0; r < T; ++r) {
      const uint64_t m = wave_min_u64(c0 < c1 ? c0 : c1);
      if (lane == 0) sh.win[r] = m;
      c0 = c0 == m ? ~0ull : c0;
      c1 = c1 == m ? ~0ull : c1;
    }
  }
  if constexpr (NW > 1) __syncthreads();
}

// Position in the selection (-1: not taken) of a thread's next valid key, in
// index order; less_before / eq_before come from block_scan2 and advance.
__device__ __forceinline__ int rank_in_selection(uint32_t key, uint32_t theta, uint32_t take_eq,
                                                 uint32_t &less_before, uint32_t &eq_before) {
  int out = -1;
  if (key < theta) {
    out = static_cast<int>(less_before + min(eq_before, take_eq));
    ++less_before;
  } else if (key == theta) {
    if (eq_before < take_eq) out = static_cast<int>(less_before + eq_before);
    ++eq_before;
  }
  return out;
}

// Updated scores of slots j0 + k * stride below lim (k < ITEMS) in every batch
// row served; rank[k] gets the ranking value.  Loads go out UB items at a time
// ahead of their stores: a store may alias a later load as far as the compiler
// knows, so interleaving them one by one would serialise ITEMS memory round trips.
template <int POL, int ITEMS>
__device__ __forceinline__ void update_scores(const EvictArgs &a, int head, int j0, int stride, int lim,
                                              float (&rank)[ITEMS]) {
  constexpr int UB = ITEMS < 8 ? ITEMS : 8;
  const int C = a.C, n_keys = a.n_occ + a.T;
  const int nb = (POL == H2O_POLICY_ORIG) ? a.B : 1;
  // ages are pos + T - token_pos; the host checks that pos + T fits in int32
  // whenever token positions are kept (and h2o_norm needs them), so the age
  // converts to fp32 with one instruction and the same rounding as from int64
  const int32_t pos_end = static_cast<int32_t>(a.pos + a.T);
  for (int bb = 0; bb < nb; ++bb) {
    const size_t g = (POL == H2O_POLICY_ORIG) ? static_cast<size_t>(bb) * a.Hkv + head : head;
    float *ph = a.scores + g * C;
    const float *wv = a.wsum + g * n_keys;
    const int32_t *tp = a.token_pos ? a.token_pos + g * C : nullptr;
#pragma unroll
    for (int k0 = 0; k0 < ITEMS; k0 += UB) {
      float f[UB], d[UB];
      int32_t t0[UB] = {};
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int j = j0 + (k0 + u) * stride;
        f[u] = j < lim ? ph[j] : 0.f;
        d[u] = j < lim ? wv[j] : 0.f;
        if constexpr (POL == H2O_POLICY_NORM) t0[u] = j < lim ? tp[j] : 0;
      }
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int k = k0 + u;
        const int j = j0 + k * stride;
        f[u] += d[u];
        if (j < lim) ph[j] = f[u];
        if constexpr (POL == H2O_POLICY_ORIG) {
          rank[k] = (bb == 0) ? f[u] : rank[k] + f[u];
        } else if constexpr (POL == H2O_POLICY_NORM) {
          rank[k] = f[u] / static_cast<float>(pos_end - t0[u]);
        } else {
          rank[k] = f[u];
        }
      }
    }
  }
}

// Replay-log entry `out` of every batch row served becomes slot j: log entry,
// score seeded with the chunk token's own sum (seed0 for the first row),
// token position.
template <int POL>
__device__ __forceinline__ void take_slot(const EvictArgs &a, int head, int j, int out, float seed0) {
  const int C = a.C, T = a.T, n_keys = a.n_occ + T;
  const int nb = (POL == H2O_POLICY_ORIG) ? a.B : 1;
  H2O_DEVICE_CHECK(j >= 0 && j < C && out >= 0 && out < T);
  for (int bb = 0; bb < nb; ++bb) {
    const size_t g = (POL == H2O_POLICY_ORIG) ? static_cast<size_t>(bb) * a.Hkv + head : head;
    const float seed = (bb == 0) ? seed0 : a.wsum[g * n_keys + C + out];
    a.slot_log[g * T + out] = j;
    a.scores[g * C + j] = seed;
    if (a.token_pos) a.token_pos[g * C + j] = static_cast<int32_t>(a.pos + out);
  }
}

// ---------------------------------------------------------------------------
// One workgroup per head: update, select, write.
// ---------------------------------------------------------------------------
template <int ITEMS, bool STAGE, int POL>
__global__ __launch_bounds__(NT) void evict_kernel(EvictArgs a) {
  // Updated scores pass through LDS so that global traffic is coalesced while
  // each thread still owns a contiguous index range (row stride ITEMS + 1
  // keeps the per-thread reads conflict-free).
  extern __shared__ float stage[];
  __shared__ SelShared sh;

  const int tid = threadIdx.x;
  const int C = a.C, T = a.T, n_occ = a.n_occ;
  const int n_keys = n_occ + T;
  const int head = blockIdx.x;  // (b, KV head); the KV head for h2o_orig
  const size_t grp0 = head;     // first batch row's group

  if (POL != H2O_POLICY_ORIG && n_occ + T <= C) {  // filling: left to right
    {
      float unused[ITEMS];
      update_scores<POL, ITEMS>(a, head, tid, NT, n_occ, unused);
    }
    const float *w = a.wsum + grp0 * n_keys;
    for (int t = tid; t < T; t += NT) {
      const int slot = n_occ + t;
      H2O_DEVICE_CHECK(slot < C);
      a.slot_log[grp0 * T + t] = slot;
      a.scores[grp0 * C + slot] = w[n_occ + t];
      if (a.token_pos) a.token_pos[grp0 * C + slot] = static_cast<int32_t>(a.pos + t);
    }
    return;
  }

  // evicting: n_occ == C
  const int base = tid * ITEMS;
  uint32_t key[ITEMS];
  if constexpr (STAGE) {  // coalesced, staged in LDS
    float f[ITEMS];
    update_scores<POL, ITEMS>(a, head, tid, NT, C, f);
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
      const int j = tid + k * NT;
      if (j < C) stage[(j / ITEMS) * (ITEMS + 1) + j % ITEMS] = f[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < ITEMS; ++k)
      key[k] = (base + k < C) ? ordered_key(stage[tid * (ITEMS + 1) + k]) : 0xffffffffu;
  } else {  // caches too large to stage: each thread reads its own range
    float f[ITEMS];
    update_scores<POL, ITEMS>(a, head, base, 1, C, f);
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) key[k] = base + k < C ? ordered_key(f[k]) : 0xffffffffu;
  }
  const int nvalid = C - base;  // items k < nvalid are slots

  uint32_t theta, take_eq;
  select_smallest<NT, ITEMS>(key, nvalid, static_cast<uint32_t>(T), sh, theta, take_eq);

  uint32_t nl = 0, ne = 0;
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) {
    if (k < nvalid) {
      nl += key[k] < theta;
      ne += key[k] == theta;
    }
  }
  uint32_t less_before, eq_before;
  block_scan2<NT>(nl, ne, less_before, eq_before, sh);
  const float *w0 = a.wsum + grp0 * n_keys;
  if constexpr (STAGE) {
    // Each taken slot goes to LDS at its position in the log (the staging
    // buffer is free: the keys are in registers); then thread i serves
    // position i, so the seeds (the chunk's own sums) are read and the log
    // written in order and only the score / position stores scatter.
    int *taken = reinterpret_cast<int *>(stage);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
      const int out = k < nvalid ? rank_in_selection(key[k], theta, take_eq, less_before, eq_before) : -1;
      if (out >= 0) taken[out] = base + k;
    }
    __syncthreads();
    for (int i = tid; i < T; i += NT) take_slot<POL>(a, head, taken[i], i, w0[C + i]);
    return;
  }
  // UB slots at a time: positions, then the batch's seeds, then its stores
  // (see update_scores)
  constexpr int UB = ITEMS < 8 ? ITEMS : 8;
#pragma unroll
  for (int k0 = 0; k0 < ITEMS; k0 += UB) {
    int out[UB];
#pragma unroll
    for (int u = 0; u < UB; ++u)
      out[u] = k0 + u < nvalid ? rank_in_selection(key[k0 + u], theta, take_eq, less_before, eq_before) : -1;
    float seed[UB];
#pragma unroll
    for (int u = 0; u < UB; ++u) seed[u] = out[u] >= 0 ? w0[C + out[u]] : 0.f;
#pragma unroll
    for (int u = 0; u < UB; ++u)
      if (out[u] >= 0) take_slot<POL>(a, head, base + k0 + u, out[u], seed[u]);
  }
}

// ---------------------------------------------------------------------------
// Short chunks, pass 1: per slice of SLICE slots, update, rank, and keep the T
// smallest (every slot of a slice that holds at most T) as (key, slot) pairs
// in slot order at cand[(head * nslice + slice) * T ..].
// ---------------------------------------------------------------------------
// The slice's candidates from its ranking keys (ITEMS per thread, slots
// base .. base + ITEMS - 1, nvalid of them real), written to dst.
template <int NTH, int ITEMS>
__device__ __forceinline__ void slice_candidates(const uint32_t (&key)[ITEMS], int base, int nvalid, int s0,
                                                 int len, int T, uint2 *dst, SelShared &sh) {
  const int tid = threadIdx.x;
  if (T == 1) {  // the slice's smallest (key, slot)
    uint64_t v = ~0ull;
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
      const uint64_t u = (static_cast<uint64_t>(key[k]) << 32) | static_cast<uint32_t>(base + k);
      if (k < nvalid && u < v) v = u;
    }
    v = block_min_u64<NTH>(v, sh.m64);
    if (tid == 0) dst[0] = make_uint2(static_cast<uint32_t>(v >> 32), static_cast<uint32_t>(v));
    return;
  }
  if (len <= T) {  // the whole slice (only the last one can be this short)
#pragma unroll
    for (int k = 0; k < ITEMS; ++k)
      if (k < nvalid) dst[base + k - s0] = make_uint2(key[k], static_cast<uint32_t>(base + k));
    return;
  }
  if (T <= SMALL_T) {
    // the slice's T smallest (key, slot), listed in increasing order (the
    // pick compares (key, slot) pairs, so list order carries no tie-break)
    uint64_t u[ITEMS];
#pragma unroll
    for (int k = 0; k < ITEMS; ++k)
      u[k] = k < nvalid ? (static_cast<uint64_t>(key[k]) << 32) | static_cast<uint32_t>(base + k) : ~0ull;
    block_smallest<NTH, ITEMS>(u, T, sh);
    if (tid < T) dst[tid] = make_uint2(static_cast<uint32_t>(sh.win[tid] >> 32), static_cast<uint32_t>(sh.win[tid]));
    return;
  }
  uint32_t rel[ITEMS];
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) rel[k] = key[k];
  uint32_t theta, take_eq;
  select_smallest<NTH, ITEMS>(rel, nvalid, static_cast<uint32_t>(T), sh, theta, take_eq);
  uint32_t nl = 0, ne = 0;
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) {
    if (k < nvalid) {
      nl += rel[k] < theta;
      ne += rel[k] == theta;
    }
  }
  uint32_t less_before, eq_before;
  block_scan2<NTH>(nl, ne, less_before, eq_before, sh);
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) {
    if (k >= nvalid) continue;
    const int out = rank_in_selection(rel[k], theta, take_eq, less_before, eq_before);
    if (out >= 0) dst[out] = make_uint2(key[k], static_cast<uint32_t>(base + k));
  }
}

template <int POL>
__global__ __launch_bounds__(NT_C) void evict_cand(EvictArgs a, uint2 *cand) {
  constexpr int ITEMS = SLICE / NT_C;
  __shared__ SelShared sh;
  const int tid = threadIdx.x;
  const int C = a.C, T = a.T;
  const int slice = blockIdx.x, head = blockIdx.y, nslice = gridDim.x;
  const int s0 = slice * SLICE;
  const int len = min(SLICE, C - s0);
  const int base = s0 + tid * ITEMS;
  const int nvalid = s0 + len - base;
  float f[ITEMS];
  update_scores<POL, ITEMS>(a, head, base, 1, s0 + len, f);
  uint32_t key[ITEMS];
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) key[k] = ordered_key(f[k]);
  slice_candidates<NT_C, ITEMS>(key, base, nvalid, s0, len, T,
                               cand + (static_cast<size_t>(head) * nslice + slice) * T, sh);
}

// Pass 1 for short chunks whose pass A stored its logits (a.lg, at most
// LOGIT_ROWS_MAX rows per group): the workgroup first forms its slice's
// summed weights from the logits -- the sum attn_b_logits forms, in the same
// order -- and writes them, so the step needs no separate weight-sum launch;
// then it updates, ranks and lists candidates as evict_cand does.  One slot
// per thread (NT_LG threads), so the sums keep the parallelism of a kernel of
// their own.  Workgroups with slice index x also merge output rows x,
// x + nslice, ... of their groups from the key splits (and write their
// normalisers), and slice 0 sums the chunk's own keys.
constexpr int NT_LG = SLICE;
template <int POL>
__global__ __launch_bounds__(NT_LG) void evict_cand_lg(EvictArgs e, AttnArgs a, float xs, uint2 *cand) {
  __shared__ SelShared sh;
  __shared__ float Ls[LOGIT_ROWS_MAX], Ms[LOGIT_ROWS_MAX], Ws[LOGIT_ROWS_MAX];
  __shared__ float4 red_o[8][32];
  const int tid = threadIdx.x;
  const int C = e.C, T = e.T;
  const int slice = blockIdx.x, head = blockIdx.y, nslice = gridDim.x;
  const int s0 = slice * SLICE;
  const int len = min(SLICE, C - s0);
  const int j = s0 + tid;  // this thread's slot
  const bool own = tid < len;
  const int R = a.qg * a.T;
  const int n_keys = C + T;  // evicting: every slot is occupied
  const int nb = (POL == H2O_POLICY_ORIG) ? e.B : 1;
  const int32_t pos_end = static_cast<int32_t>(e.pos + T);
  const size_t rows = static_cast<size_t>(a.B) * a.Hq * a.T;
  const bool merger = a.nsplit > 1 && tid < 256;  // 8 groups of 32 lanes merge output rows
  const int q8 = (tid >> 5) & 7, c4 = tid & 31;
  const int rn = tid >> 4, sl = tid & 15;  // normalisers: 16 lanes per row
  // h2o_orig, which loops over the batch rows, loads a merged row's partials
  // only when it merges it (registers)
  constexpr bool kEarlyRow = POL != H2O_POLICY_ORIG;
  float rank = 0.f;
  for (int bb = 0; bb < nb; ++bb) {
    const int grp = (POL == H2O_POLICY_ORIG) ? bb * e.Hkv + head : head;
    const int g = grp % a.Hkv, b = grp / a.Hkv;
    auto row_index = [&](int r) {
      return (static_cast<size_t>(b) * a.Hq + g * a.qg + r % a.qg) * a.T + r / a.qg;
    };
    // Every load of the group first (none depends on another): split (m, l)
    // pairs, the first merged row's partials, the slot's logits, score and
    // token position.
    float2 ml[4];
    load_split_ml(a, rows, rn < R ? row_index(rn) : 0, sl, a.nsplit > 1 && rn < R, ml);
    const float lse_own = (a.nsplit == 1 && tid < R) ? a.lse2[row_index(tid)] : 0.f;
    float ms[8];
    float4 po[8];
    if (kEarlyRow && slice < R) load_split_row(a, rows, row_index(slice), q8, c4, merger, ms, po);
    const float *lgp = a.lg + static_cast<size_t>(grp) * R * a.lg_stride;
    float x[LOGIT_ROWS_MAX];
#pragma unroll
    for (int r = 0; r < LOGIT_ROWS_MAX; ++r) x[r] = (r < R && own) ? lgp[static_cast<size_t>(r) * a.lg_stride + j] : 0.f;
    float *ph = e.scores + static_cast<size_t>(grp) * C;
    float f = own ? ph[j] : 0.f;
    int32_t t0 = 0;
    if constexpr (POL == H2O_POLICY_NORM) t0 = own ? e.token_pos[static_cast<size_t>(grp) * C + j] : 0;

    // row normalisers of the group: merged from the key splits, or pass A's own
    if (a.nsplit > 1) {
      float M, W;
      reduce_split_ml(ml, M, W);
      if (rn < R && sl == 0) {
        Ms[rn] = M;
        Ws[rn] = W;
        Ls[rn] = M + log2f(W);
      }
    } else if (tid < R) {
      Ls[tid] = lse_own;
    }
    __syncthreads();
    for (int r = slice; a.nsplit > 1 && r < R; r += nslice) {
      const size_t li = row_index(r);
      if (!kEarlyRow || r != slice) load_split_row(a, rows, li, q8, c4, merger, ms, po);
      merge_split_row(a, li, Ms[r], Ws[r], Ls[r], q8, c4, merger, ms, po, red_o);
      __syncthreads();  // red_o is reused by the next row
    }
    // summed weights: every row sees the cache slots, row r sees chunk key t
    // iff t * q_g <= r - r % q_g
    float *w = a.wsum + static_cast<size_t>(grp) * n_keys;
    const float d = key_weight_sum(R, [&](int r) { return x[r]; }, [](int) { return true; }, xs, Ls);
    if (slice == 0 && tid < T) {  // chunk key tid: its logits into x, all loads first
#pragma unroll
      for (int r = 0; r < LOGIT_ROWS_MAX; ++r) x[r] = r < R ? lgp[static_cast<size_t>(r) * a.lg_stride + C + tid] : 0.f;
      w[C + tid] = key_weight_sum(
          R, [&](int r) { return x[r]; }, [&](int r) { return tid * a.qg <= r - r % a.qg; }, xs, Ls);
    }
    if (own) {
      w[j] = d;
      f += d;
      ph[j] = f;
      if constexpr (POL == H2O_POLICY_ORIG) {
        rank = (bb == 0) ? f : rank + f;
      } else if constexpr (POL == H2O_POLICY_NORM) {
        rank = f / static_cast<float>(pos_end - t0);
      } else {
        rank = f;
      }
    }
    __syncthreads();  // Ls / Ms / Ws are rewritten for the next batch row
  }
  const uint32_t key[1] = {own ? ordered_key(rank) : 0xffffffffu};
  slice_candidates<NT_LG, 1>(key, j, own ? 1 : 0, s0, len, T, cand + (static_cast<size_t>(head) * nslice + slice) * T,
                             sh);
}

// Short chunks, pass 2: the T smallest candidates of each head.  The lists
// of the slices follow one another in slot order, so list order breaks ties
// as slot order does.  ncand: list length per head (the last slice may fill
// fewer than T entries: nreal counts the filled ones, which come first).
//
// KV: also write the chunk's K and V rows into the slots this head took,
// replacing the separate write kernel for short chunks: the slots stay in
// LDS, and the rows of T <= KV_FUSE_T tokens are a few KB per head.  Native
// caches copy the rows; 8/4-bit caches (one token) quantise them, one
// wavefront per row, with the write kernel's own row quantiser.
template <int NTH, int ITEMS, int POL, bool KV>
__global__ __launch_bounds__(NTH) void evict_pick(EvictArgs a, const uint2 *cand, int ncand, int nreal,
                                                 KvWriteArgs kv) {
  __shared__ SelShared sh;
  __shared__ int chosen[KV ? KV_FUSE_T : 1];
  const int tid = threadIdx.x;
  const int C = a.C, T = a.T, n_keys = a.n_occ + T;
  const int head = blockIdx.x;
  auto write_rows = [&]() {
    __syncthreads();  // chosen[] complete
    const int nb = (POL == H2O_POLICY_ORIG) ? a.B : 1;
    if (kv.cache_fmt != FMT_NATIVE) {  // bf16 rows: one wavefront per (batch row, token, K or V)
      const int lane = tid & 63;
      for (int r = tid >> 6; r < nb * T * 2; r += NTH / 64) {
        const int isv = r & 1, t = (r >> 1) % T, bb = (r >> 1) / T;
        const size_t g = (POL == H2O_POLICY_ORIG) ? static_cast<size_t>(bb) * a.Hkv + head : head;
        const size_t dst_row = g * C + chosen[t];
        if (kv.cache_fmt == FMT_INT8) {
          quantize_row<DT_BF16, FMT_INT8>(kv, g * T + t, dst_row, isv, lane);
        } else {
          quantize_row<DT_BF16, FMT_INT4>(kv, g * T + t, dst_row, isv, lane);
        }
      }
      return;
    }
    const int row_bytes = kv.D * (kv.dtype == DT_F32 ? 4 : 2);
    const int cpr = row_bytes / 16;
    const int total = nb * T * 2 * cpr;
    for (int i = tid; i < total; i += NTH) {
      const int chunk = i % cpr;
      int rest = i / cpr;
      const int isv = rest & 1;
      rest >>= 1;
      const int t = rest % T, bb = rest / T;
      const size_t g = (POL == H2O_POLICY_ORIG) ? static_cast<size_t>(bb) * a.Hkv + head : head;
      const char *src = static_cast<const char *>(isv ? kv.vn : kv.kn) + (g * T + t) * row_bytes + chunk * 16;
      char *dst = static_cast<char *>(isv ? kv.vc : kv.kc) + (g * C + chosen[t]) * row_bytes + chunk * 16;
      *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
    }
  };
  const uint2 *src = cand + static_cast<size_t>(head) * ncand;
  const int base = tid * ITEMS;
  const int nvalid = nreal - base;
  uint32_t key[ITEMS];
  int slot[ITEMS];
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) {
    const uint2 c = k < nvalid ? src[base + k] : make_uint2(0xffffffffu, 0u);
    key[k] = c.x;
    slot[k] = static_cast<int>(c.y);
  }
  if (T == 1) {
    uint64_t v = ~0ull;
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
      const uint64_t u = (static_cast<uint64_t>(key[k]) << 32) | static_cast<uint32_t>(slot[k]);
      if (k < nvalid && u < v) v = u;
    }
    v = block_min_u64<NTH>(v, sh.m64);
    if (tid == 0) {
      const int j = static_cast<int>(static_cast<uint32_t>(v));
      take_slot<POL>(a, head, j, 0, a.wsum[static_cast<size_t>(head) * n_keys + C]);
      if constexpr (KV) chosen[0] = j;
    }
    if constexpr (KV) write_rows();
    return;
  }
  if (T <= SMALL_T) {
    // the T smallest (key, slot); each winner's place in slot order is the
    // number of winners with a lower slot
    uint64_t u[ITEMS];
#pragma unroll
    for (int k = 0; k < ITEMS; ++k)
      u[k] = k < nvalid ? (static_cast<uint64_t>(key[k]) << 32) | static_cast<uint32_t>(slot[k]) : ~0ull;
    block_smallest<NTH, ITEMS>(u, T, sh);
    if (tid < T) {
      const uint32_t j = static_cast<uint32_t>(sh.win[tid]);
      int out = 0;
      for (int r = 0; r < T; ++r) out += static_cast<uint32_t>(sh.win[r]) < j;
      take_slot<POL>(a, head, static_cast<int>(j), out, a.wsum[static_cast<size_t>(head) * n_keys + C + out]);
      if constexpr (KV) chosen[out] = static_cast<int>(j);
    }
    if constexpr (KV) write_rows();
    return;
  }
  uint32_t theta, take_eq;
  select_smallest<NTH, ITEMS>(key, nvalid, static_cast<uint32_t>(T), sh, theta, take_eq);
  uint32_t nl = 0, ne = 0;
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) {
    if (k < nvalid) {
      nl += key[k] < theta;
      ne += key[k] == theta;
    }
  }
  uint32_t less_before, eq_before;
  block_scan2<NTH>(nl, ne, less_before, eq_before, sh);
  const float *w0 = a.wsum + static_cast<size_t>(head) * n_keys;
  constexpr int UB = ITEMS < 8 ? ITEMS : 8;  // as in evict_kernel
#pragma unroll
  for (int k0 = 0; k0 < ITEMS; k0 += UB) {
    int out[UB];
#pragma unroll
    for (int u = 0; u < UB; ++u)
      out[u] = k0 + u < nvalid ? rank_in_selection(key[k0 + u], theta, take_eq, less_before, eq_before) : -1;
    float seed[UB];
#pragma unroll
    for (int u = 0; u < UB; ++u) seed[u] = out[u] >= 0 ? w0[C + out[u]] : 0.f;
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      if (out[u] >= 0) {
        take_slot<POL>(a, head, slot[k0 + u], out[u], seed[u]);
        if constexpr (KV) chosen[out[u]] = slot[k0 + u];
      }
    }
  }
  if constexpr (KV) write_rows();
}

template <int ITEMS, int POL>
hipError_t launch_pol(const EvictArgs &a, hipStream_t s) {
  constexpr bool STAGE = ITEMS <= 32;  // 1024 x 33 floats = 132 KB of LDS at most
  constexpr int stage_bytes = STAGE ? static_cast<int>(sizeof(float)) * NT * (ITEMS + 1) : 0;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void *>(&evict_kernel<ITEMS, STAGE, POL>),
      hipFuncAttributeMaxDynamicSharedMemorySize, stage_bytes);
  if (attr != hipSuccess) return attr;
  const bool evicting = a.n_occ == a.C;
  const size_t lds = evicting ? stage_bytes : 0;
  const int grid = (POL == H2O_POLICY_ORIG) ? a.Hkv : a.groups;
  KernelTimer timer(H2O_K_EVICT, s);
  hipLaunchKernelGGL((evict_kernel<ITEMS, STAGE, POL>), dim3(grid), dim3(NT), lds, s, a);
  return hipGetLastError();
}

template <int ITEMS>
hipError_t launch_items(const EvictArgs &a, hipStream_t s) {
  // Filling is the same under every policy.
  if (a.n_occ + a.T <= a.C || a.policy == H2O_POLICY_H2O) return launch_pol<ITEMS, H2O_POLICY_H2O>(a, s);
  if (a.policy == H2O_POLICY_NORM) return launch_pol<ITEMS, H2O_POLICY_NORM>(a, s);
  return launch_pol<ITEMS, H2O_POLICY_ORIG>(a, s);
}

int n_slices(int C) { return (C + SLICE - 1) / SLICE; }

// Candidate lists of at most half the slots: the two-pass shape pays off.
bool two_pass_fits(int C, int T) { return 2LL * n_slices(C) * T <= C; }

template <int POL, bool KV>
void launch_pick(const EvictArgs &a, const uint2 *cand, int ncand, int nreal, const KvWriteArgs &kv,
                 int heads, hipStream_t s) {
  // short lists: one wavefront (two when the pick quantises a K and a V
  // row per head); longer ones: 256 or 1024 threads
  if (KV && kv.cache_fmt != FMT_NATIVE && a.T == 1 && nreal <= 128) {
    hipLaunchKernelGGL((evict_pick<128, 1, POL, KV>), dim3(heads), dim3(128), 0, s, a, cand, ncand, nreal, kv);
  } else if (KV && kv.cache_fmt != FMT_NATIVE && nreal <= 512) {  // a wavefront per quantised row
    hipLaunchKernelGGL((evict_pick<512, 1, POL, KV>), dim3(heads), dim3(512), 0, s, a, cand, ncand, nreal, kv);
  } else if (nreal <= 64) {
    hipLaunchKernelGGL((evict_pick<64, 1, POL, KV>), dim3(heads), dim3(64), 0, s, a, cand, ncand, nreal, kv);
  } else if (nreal <= 256) {
    hipLaunchKernelGGL((evict_pick<64, 4, POL, KV>), dim3(heads), dim3(64), 0, s, a, cand, ncand, nreal, kv);
  } else if (nreal <= 1024) {
    hipLaunchKernelGGL((evict_pick<256, 4, POL, KV>), dim3(heads), dim3(256), 0, s, a, cand, ncand, nreal, kv);
  } else if (nreal <= 4096) {
    hipLaunchKernelGGL((evict_pick<256, 16, POL, KV>), dim3(heads), dim3(256), 0, s, a, cand, ncand, nreal, kv);
  } else if (nreal <= 16384) {
    hipLaunchKernelGGL((evict_pick<NT, 16, POL, KV>), dim3(heads), dim3(NT), 0, s, a, cand, ncand, nreal, kv);
  } else {
    hipLaunchKernelGGL((evict_pick<NT, 32, POL, KV>), dim3(heads), dim3(NT), 0, s, a, cand, ncand, nreal, kv);
  }
}

// kv: when set, the pick also writes the chunk's K/V rows.  lg: when set,
// the candidate pass also forms the summed weights from the stored logits.
template <int POL>
hipError_t launch_two_pass(const EvictArgs &a, uint2 *cand, const KvWriteArgs *kv, const AttnArgs *lg,
                           hipStream_t s) {
  const int heads = (POL == H2O_POLICY_ORIG) ? a.Hkv : a.groups;
  const int ns = n_slices(a.C);
  const int ncand = ns * a.T;
  const int last = a.C - (ns - 1) * SLICE;  // slots of the last slice
  const int nreal = (ns - 1) * a.T + (last < a.T ? last : a.T);
  KernelTimer timer(H2O_K_EVICT, s);
  if (lg) {
    const float xs = lg->cache_fmt == FMT_NATIVE ? lg->sl2 : 1.f;
    hipLaunchKernelGGL(evict_cand_lg<POL>, dim3(ns, heads), dim3(NT_LG), 0, s, a, *lg, xs, cand);
  } else {
    hipLaunchKernelGGL(evict_cand<POL>, dim3(ns, heads), dim3(NT_C), 0, s, a, cand);
  }
  if (kv) {
    launch_pick<POL, true>(a, cand, ncand, nreal, *kv, heads, s);
  } else {
    launch_pick<POL, false>(a, cand, ncand, nreal, KvWriteArgs{}, heads, s);
  }
  return hipGetLastError();
}

}  // namespace

size_t evict_workspace_bytes(int groups, int C, int T) {
  if (!two_pass_fits(C, T)) return 0;
  return sizeof(uint2) * static_cast<size_t>(groups) * n_slices(C) * T;
}

bool evict_two_pass(const EvictArgs &a, size_t ws_bytes) {
  const size_t need = evict_workspace_bytes(a.groups, a.C, a.T);
  return a.n_occ == a.C && need && ws_bytes >= need;
}

hipError_t launch_evict(const EvictArgs &a, void *ws, size_t ws_bytes, hipStream_t s, const KvWriteArgs *kv,
                        bool *kv_done, const AttnArgs *lg) {
  if (kv_done) *kv_done = false;
  if (ws && evict_two_pass(a, ws_bytes)) {
    uint2 *cand = static_cast<uint2 *>(ws);
    // stored logits: short chunks (at most LOGIT_ROWS_MAX query rows per
    // group), bf16 queries, D = 128, buffers matching the selection's
    if (lg && (!lg->lg || !lg->wsum || lg->D != 128 || lg->qg * lg->T > LOGIT_ROWS_MAX ||
               lg->B * lg->Hkv != a.groups || lg->T != a.T || lg->n_occ != a.n_occ || lg->nsplit > 64))
      return hipErrorInvalidValue;
    // fuse the K/V write into the pick (evict-only bookkeeping): native
    // caches up to KV_FUSE_T tokens; 8/4-bit caches up to QKV_FUSE_T tokens,
    // whose 2T quantised rows per head the pick's wavefronts take one each
    // (with T = 1 a two-wavefront pick; else eight)
    const bool fuse = kv && kv_done && !kv->token_pos &&
                      ((kv->cache_fmt == FMT_NATIVE && a.T <= KV_FUSE_T) ||
                       (kv->dtype == DT_BF16 && a.T <= QKV_FUSE_T && kv->D <= 128 &&
                        n_slices(a.C) * a.T <= 512));
    const KvWriteArgs *kvp = fuse ? kv : nullptr;
    if (fuse) *kv_done = true;
    if (a.policy == H2O_POLICY_NORM) return launch_two_pass<H2O_POLICY_NORM>(a, cand, kvp, lg, s);
    if (a.policy == H2O_POLICY_ORIG) return launch_two_pass<H2O_POLICY_ORIG>(a, cand, kvp, lg, s);
    return launch_two_pass<H2O_POLICY_H2O>(a, cand, kvp, lg, s);
  }
  if (lg) return hipErrorInvalidValue;  // only the candidate pass sums stored logits
  const int per = (a.C + NT - 1) / NT;
  if (per <= 1) return launch_items<1>(a, s);
  if (per <= 2) return launch_items<2>(a, s);
  if (per <= 4) return launch_items<4>(a, s);
  if (per <= 8) return launch_items<8>(a, s);
  if (per <= 16) return launch_items<16>(a, s);
  if (per <= 32) return launch_items<32>(a, s);
  return launch_items<64>(a, s);
}

}  // namespace h2o
