// Score accumulate + slot selection + replay log + seeding, one workgroup of
// 1024 threads per (b, KV head) -- per KV head for h2o_orig.
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
// radix select over the order-preserving uint32 image of the fp32 scores
// (4 passes of 8 bits, LDS histograms with wave-aggregated increments), then
// an index-ordered compaction: a slot is taken if its key is below the
// threshold key, or equal to it and among the first k such slots.  The replay
// log row comes out in ascending slot order; chunk token t goes to the t-th
// entry.  Each thread owns ITEMS consecutive slots held in registers (loaded
// through LDS so that global accesses stay coalesced).

#include "device_util.hpp"
#include "h2o_internal.hpp"

namespace h2o {
namespace {

constexpr int NT = 1024;
constexpr int NWAVES = NT / 64;

__device__ __forceinline__ uint32_t ordered_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0 ranks with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Block-wide exclusive scan of two counters; returns the prefixes for this thread.
__device__ __forceinline__ void block_scan2(uint32_t a, uint32_t b, uint32_t &ea, uint32_t &eb,
                                            uint32_t *sh_a, uint32_t *sh_b) {
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
    sh_a[wave] = ia;
    sh_b[wave] = ib;
  }
  __syncthreads();
  uint32_t pa = 0, pb = 0;
  for (int w = 0; w < wave; ++w) {
    pa += sh_a[w];
    pb += sh_b[w];
  }
  ea = pa + ia - a;
  eb = pb + ib - b;
}

template <int ITEMS, bool STAGE, int POL>
__global__ __launch_bounds__(NT) void evict_kernel(EvictArgs a) {
  // Updated scores pass through LDS so that global traffic is coalesced while
  // each thread still owns a contiguous index range (row stride ITEMS + 1
  // keeps the per-thread reads conflict-free).
  extern __shared__ float stage[];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh_sel, sh_k;
  __shared__ uint32_t sh_a[NWAVES], sh_b[NWAVES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int C = a.C, T = a.T, n_occ = a.n_occ;
  const int n_keys = n_occ + T;
  // h2o_orig: this workgroup serves KV head blockIdx.x of every batch row
  const int nb = (POL == H2O_POLICY_ORIG) ? a.B : 1;
  auto grp_of = [&](int bb) { return (POL == H2O_POLICY_ORIG) ? bb * a.Hkv + blockIdx.x : blockIdx.x; };
  const int grp = grp_of(0);
  float *phi = a.scores + static_cast<size_t>(grp) * C;
  const float *w = a.wsum + static_cast<size_t>(grp) * n_keys;
  int32_t *log = a.slot_log + static_cast<size_t>(grp) * T;
  int32_t *tp = a.token_pos ? a.token_pos + static_cast<size_t>(grp) * C : nullptr;
  // Updated score of slot j in every batch row served; returns the ranking value.
  auto update = [&](int j) -> float {
    if constexpr (POL == H2O_POLICY_ORIG) {
      float tot = 0.f;
      for (int bb = 0; bb < nb; ++bb) {
        const size_t g = static_cast<size_t>(grp_of(bb));
        const float f = a.scores[g * C + j] + a.wsum[g * n_keys + j];
        a.scores[g * C + j] = f;
        tot = (bb == 0) ? f : tot + f;
      }
      return tot;
    } else {
      const float f = phi[j] + w[j];
      phi[j] = f;
      if constexpr (POL == H2O_POLICY_NORM) {
        return f / static_cast<float>(a.pos + T - tp[j]);
      }
      return f;
    }
  };

  if (POL != H2O_POLICY_ORIG && n_occ + T <= C) {  // filling: left to right
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
      const int j = tid + k * NT;
      if (j < n_occ) phi[j] = phi[j] + w[j];
    }
    for (int t = tid; t < T; t += NT) {
      const int slot = n_occ + t;
      log[t] = slot;
      phi[slot] = w[n_occ + t];
      if (tp) tp[slot] = static_cast<int32_t>(a.pos + t);
    }
    return;
  }

  // evicting: n_occ == C.  phi += w
  const int base = tid * ITEMS;
  uint32_t key[ITEMS];
  if constexpr (STAGE) {  // coalesced, staged in LDS
    // fixed trip count so that all loads of a thread are in flight together
    float f[ITEMS];
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
      const int j = tid + k * NT;
      f[k] = (j < C) ? update(j) : 0.f;
    }
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
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
      const int j = base + k;
      key[k] = 0xffffffffu;
      if (j < C) key[k] = ordered_key(update(j));
    }
  }

  // Keys relative to the block minimum, so that the first 8-bit digit is
  // taken from the top of the occupied range (the raw top byte -- sign and
  // exponent -- takes few values, and counting them serialises on a few bins).
  {
    uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
      if (base + k < C) {
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
      sh_a[tid >> 6] = kmin;
      sh_b[tid >> 6] = kmax;
    }
    __syncthreads();
    kmin = sh_a[0];
    kmax = sh_b[0];
    for (int wv = 1; wv < NWAVES; ++wv) {
      kmin = min(kmin, sh_a[wv]);
      kmax = max(kmax, sh_b[wv]);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) key[k] -= kmin;  // padding keys wrap to large values, never active
    const uint32_t range = kmax - kmin;
    sh_k = range ? 32 - __builtin_clz(range) : 0;  // significant bits of the range
  }
  __syncthreads();
  const int nbits = static_cast<int>(sh_k);
  __syncthreads();
  const int npass = (nbits + 7) / 8;

  uint32_t prefix = 0, pmask = 0, need = static_cast<uint32_t>(T);
  for (int pass = 0; pass < npass; ++pass) {
    // digit p covers bits [shift, shift + width) counted from the top of the range
    int shift = nbits - 8 * (pass + 1), width = 8;
    if (shift < 0) {
      width += shift;
      shift = 0;
    }
    const uint32_t dmask = (1u << width) - 1u;
    for (int e = tid; e < 256; e += NT) hist[e] = 0;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
      const bool act = (base + k < C) && ((key[k] & pmask) == prefix);
      const uint32_t digit = (key[k] >> shift) & dmask;
      // one LDS atomic per key; lanes hitting the same bin are serialised by
      // the LDS, which costs less than aggregating per distinct digit
      if (act) atomicAdd(&hist[digit], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      const uint32_t c0 = hist[4 * tid], c1 = hist[4 * tid + 1];
      const uint32_t c2 = hist[4 * tid + 2], c3 = hist[4 * tid + 3];
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
        sh_sel = d;
        sh_k = need - c;
      }
    }
    __syncthreads();
    prefix |= sh_sel << shift;
    pmask |= dmask << shift;
    need = sh_k;
    __syncthreads();
  }
  const uint32_t theta = prefix;  // key of the T-th smallest slot
  const uint32_t take_eq = need;  // how many slots with key == theta are taken

  uint32_t nl = 0, ne = 0;
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) {
    if (base + k < C) {
      nl += key[k] < theta;
      ne += key[k] == theta;
    }
  }
  uint32_t less_before, eq_before;
  block_scan2(nl, ne, less_before, eq_before, sh_a, sh_b);
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) {
    const int j = base + k;
    if (j >= C) break;
    int out = -1;
    if (key[k] < theta) {
      out = static_cast<int>(less_before + min(eq_before, take_eq));
      ++less_before;
    } else if (key[k] == theta) {
      if (eq_before < take_eq) out = static_cast<int>(less_before + eq_before);
      ++eq_before;
    }
    if (out >= 0) {
      for (int bb = 0; bb < nb; ++bb) {
        const size_t g = static_cast<size_t>(grp_of(bb));
        a.slot_log[g * T + out] = j;
        a.scores[g * C + j] = a.wsum[g * n_keys + C + out];
        if (a.token_pos) a.token_pos[g * C + j] = static_cast<int32_t>(a.pos + out);
      }
    }
  }
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

}  // namespace

hipError_t launch_evict(const EvictArgs &a, hipStream_t s) {
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
