// Pass A for 8-bit and 4-bit caches with head dimension 128 on gfx950.
//
// Same mathematics as the other attention passes ("Learning how to Forget",
// §A.7: softmax of mask(d_h^{-1/2} Q K^T), output Y = m V; §A.1 mask with the
// chunk attending before it is written), with the cache read as codes:
// int8 x = c*s, int4 x = c*s + z, per slot.  Codes are exact in bf16, so the
// matrix products run on the codes and the per-slot factors are applied
// outside them:
//   logit_ij = s_j <q_i, c_j> (+ z_j sum(q_i))
//   out_i    = sum_j (P_ij s_j) c_j (+ sum_j P_ij z_j, the same for every d)
//
// Per 64-key tile: the codes (8 KB int8 / 4 KB int4 per K or V tile) and the
// fp16 factors move HBM -> LDS by buffer-load DMA one tile ahead into two
// staging slots; the four wavefronts then widen the codes of the current tile
// into bf16 K and V tiles in the swizzled layouts the MFMA operand reads use,
// and compute S^T = K Q^T, the online softmax and O^T += V^T P^T as the
// native kernel does.  Chunk keys (the new tokens, bf16 inputs) are copied
// into the bf16 tiles directly.  Quantised caches are mainly read at small
// chunk lengths, where the step is bound by HBM: the codes halve or quarter
// the bytes moved.

#include <type_traits>

#include "device_util.hpp"
#include "h2o_internal.hpp"
#include "tile_util.hpp"

namespace h2o {
namespace {

typedef float f32x8 __attribute__((ext_vector_type(8)));

// Workgroup barrier that waits for this wavefront's LDS operations but not
// for its outstanding DMA (__syncthreads() would wait for both).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((63 & 15) | ((63 >> 4) << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Orders LDS accesses between the lanes of one wavefront.  A wavefront's LDS
// instructions execute in issue order, so no wait is needed: the fences only
// keep the compiler from moving memory operations across this point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int FMT>
struct QTile {
  static constexpr int CODE_ROW = (FMT == FMT_INT8) ? 128 : 64;  // bytes of codes per key
  static constexpr int CODE_BYTES = 64 * CODE_ROW;                // per K or V tile
  static constexpr int SEGS = CODE_BYTES / 1024;                  // 1 KB DMA segments per tile
  static constexpr int NFAC = (FMT == FMT_INT8) ? 2 : 4;          // fp16 factor rows: ks, vs (, kz, vz)
};

// 32 codes starting at element 32*q of a key row -> 32 bf16 (4 x 16 bytes).
template <int FMT>
__device__ __forceinline__ void widen32(const char *codes, uint4 (&out)[4]) {
  if constexpr (FMT == FMT_INT8) {
    const uint4 a = *reinterpret_cast<const uint4 *>(codes);
    const uint4 b = *reinterpret_cast<const uint4 *>(codes + 16);
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t r[4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int32_t x = static_cast<int32_t>(w[2 * i + h]);
        // integers are exact in bf16: the top half of the fp32 value is the bf16
        const float f0 = static_cast<float>((x << 24) >> 24), f1 = static_cast<float>((x << 16) >> 24);
        const float f2 = static_cast<float>((x << 8) >> 24), f3 = static_cast<float>(x >> 24);
        r[2 * h] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
        r[2 * h + 1] = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
      }
      out[i] = make_uint4(r[0], r[1], r[2], r[3]);
    }
  } else {
    const uint4 a = *reinterpret_cast<const uint4 *>(codes);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // even elements are the low nibbles, odd ones the high nibbles; with the
      // nibbles spread into bytes each converts with one v_cvt_f32_ubyteN
      const uint32_t ev = w[i] & 0x0f0f0f0fu, od = (w[i] >> 4) & 0x0f0f0f0fu;
      uint32_t r[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float lo = static_cast<float>((ev >> (8 * q)) & 0xffu);
        const float hi = static_cast<float>((od >> (8 * q)) & 0xffu);
        r[q] = __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
      }
      out[i] = make_uint4(r[0], r[1], r[2], r[3]);
    }
  }
}

// LG: also store every tile's logits (in log2 units) for short chunks (a.lg).
// NW: wavefronts per block (4 or 8), 32 rows each; a widened tile serves them all.
template <int FMT, bool LG, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void attn_a_quant(AttnArgs a) {
  constexpr int ROWS = 32 * NW;
  using Q = QTile<FMT>;
  // bf16 tiles: two with 8 wavefronts (one block per CU), so that tile t+1 is
  // widened beside the compute of tile t; one with 4 (two blocks per CU)
  constexpr int NB = NW == 8 ? 2 : 1;
  __shared__ __attribute__((aligned(1024))) char kbs[NB][TILE_BYTES];  // bf16 K tile (K/Q swizzle)
  __shared__ __attribute__((aligned(1024))) char vbs[NB][TILE_BYTES];  // bf16 V tile (V swizzle)
  __shared__ __attribute__((aligned(1024))) char kc0[Q::CODE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vc0[Q::CODE_BYTES];
  __shared__ __attribute__((aligned(1024))) char kc1[Q::CODE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vc1[Q::CODE_BYTES];
  __shared__ __attribute__((aligned(256))) uint16_t fc0[Q::NFAC][64];  // fp16 factors, slot 0
  __shared__ __attribute__((aligned(256))) uint16_t fc1[Q::NFAC][64];  // fp16 factors, slot 1
  // factors of a widened tile: [0] sl2*s_k, [1] sl2*z_k, [2] s_v, [3] z_v (chunk keys: sl2, 0, 1, 0)
  __shared__ __attribute__((aligned(256))) float facs[NB][4][64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, hl = lane >> 5;
  const int R = a.qg * a.T;
  const int tiles_per_grp = (R + ROWS - 1) / ROWS;
  const int wi_all = xcd_remap(blockIdx.x, gridDim.x);
  const int split = wi_all % a.nsplit;
  const int wi = wi_all / a.nsplit;
  // Row blocks go out last first: under the causal mask the last rows see the
  // most keys, and starting the longest blocks first evens out the tail.
  const int grp = wi / tiles_per_grp, rt = tiles_per_grp - 1 - wi % tiles_per_grp;
  const int g = grp % a.Hkv, b = grp / a.Hkv;
  const int row0 = rt * ROWS;
  const int wrow0 = row0 + wave * 32;
  const int my_row = wrow0 + n;
  const bool row_ok = my_row < R;
  const int i_q = row_ok ? my_row / a.qg : 0;
  const int h_q = g * a.qg + (row_ok ? my_row % a.qg : 0);
  const int n_occ = a.n_occ;
  const int wave_i_min = wrow0 / a.qg;
  const bool wave_ragged = wrow0 + 31 >= R;

  bf16x8 qf[8];
  float qsum = 0.f;
  {
    const uint16_t *qrow =
        static_cast<const uint16_t *>(a.q) + ((static_cast<size_t>(b) * a.Hq + h_q) * a.T + i_q) * D;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row_ok) v = *reinterpret_cast<const uint4 *>(qrow + 16 * st + 8 * hl);
      qf[st] = __builtin_bit_cast(bf16x8, v);
      if constexpr (FMT == FMT_INT4) {
#pragma unroll
        for (int e = 0; e < 8; ++e) qsum += static_cast<float>(qf[st][e]);
      }
    }
    if constexpr (FMT == FMT_INT4) qsum += __shfl_xor(qsum, 32);
  }

  const int last_row = min(R, row0 + ROWS) - 1;
  const int key_end = n_occ + last_row / a.qg + 1;
  const int ntiles_all = (key_end + 63) / 64;
  const int per_split = (ntiles_all + a.nsplit - 1) / a.nsplit;
  const int t_lo = split * per_split;
  const int ntiles = min(ntiles_all, t_lo + per_split) - t_lo;  // <= 0: empty split
  const size_t cache_row0 = static_cast<size_t>(grp) * a.C;
  const size_t new_row0 = static_cast<size_t>(grp) * a.T;

  // ---- DMA of a tile's codes and factors (cache rows only) ----
  const rsrc_t kc_rs = make_rsrc(static_cast<const char *>(a.kc) + cache_row0 * Q::CODE_ROW,
                                 n_occ * Q::CODE_ROW);
  const rsrc_t vc_rs = make_rsrc(static_cast<const char *>(a.vc) + cache_row0 * Q::CODE_ROW,
                                 n_occ * Q::CODE_ROW);
  const uint16_t *fsrc[4] = {a.ks, a.vs, a.kz, a.vz};
  // Rows past n_occ (in the one tile that may straddle it) must not be read:
  // that tile gets resources that start at its first row and end at n_occ,
  // so the range check turns those lanes into zeros.
  auto issue_codes = [&](int tile, char *kdst, char *vdst, uint16_t (*fdst)[64]) {
    const int j0 = (t_lo + tile) * 64;
    if (j0 >= n_occ) return;  // chunk keys come from the bf16 inputs
    const bool whole = j0 + 64 <= n_occ;
    const uint32_t rows_left = static_cast<uint32_t>(n_occ - j0);
    const rsrc_t kr = whole ? kc_rs
                            : make_rsrc(static_cast<const char *>(a.kc) + (cache_row0 + j0) * Q::CODE_ROW,
                                        rows_left * Q::CODE_ROW);
    const rsrc_t vr = whole ? vc_rs
                            : make_rsrc(static_cast<const char *>(a.vc) + (cache_row0 + j0) * Q::CODE_ROW,
                                        rows_left * Q::CODE_ROW);
    const uint32_t soff = whole ? static_cast<uint32_t>(j0 * Q::CODE_ROW) : 0u;
    for (int sgm = wave; sgm < Q::SEGS; sgm += NW) {
      const uint32_t off = static_cast<uint32_t>(sgm * 1024 + 16 * lane);
      dma16(kr, off, soff, kdst + sgm * 1024);
      dma16(vr, off, soff, vdst + sgm * 1024);
    }
    if (wave < Q::NFAC && lane < 32) {
      const rsrc_t fr = make_rsrc(fsrc[wave] + cache_row0 + j0, rows_left * 2);
      dma4(fr, 4 * lane, 0, reinterpret_cast<char *>(fdst[wave]));
    }
  };

  // ---- codes (or chunk rows) of the current tile -> bf16 tiles, factors ----
  // Thread tid widens the 32-element quarter tid % 4 of key row (tid % 256) / 4:
  // of K and V with 4 wavefronts, of K (wavefronts 0-3) or V (4-7) with 8.
  const int crow = (tid & 255) >> 2, cq = tid & 3;
  auto widen_rows = [&](int j, const char *cs, const void *nsrc, char *dst, bool is_v) {
    uint4 w[4];
    if (j < n_occ) {
      widen32<FMT>(cs + crow * Q::CODE_ROW + cq * (Q::CODE_ROW / 4), w);
    } else {
      const int t = j - n_occ;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w[i] = make_uint4(0, 0, 0, 0);
        if (t < a.T) w[i] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(nsrc) +
                                                               (new_row0 + t) * D + 32 * cq + 8 * i);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4 *>(dst + (is_v ? v_off(crow, 4 * cq + i) : kq_off(crow, 4 * cq + i))) = w[i];
  };
  auto widen_tile = [&](int tile, const char *kcs, const char *vcs, const uint16_t (*fcs)[64], char *kb,
                        char *vb, float (*fac)[64]) {
    const int j0 = (t_lo + tile) * 64;
    const int j = j0 + crow;
    if (NW == 4 || wave < 4) widen_rows(j, kcs, a.kn, kb, false);
    if (NW == 4 || wave >= 4) widen_rows(j, vcs, a.vn, vb, true);
    if (tid < 64) {
      const bool cached = j0 + tid < n_occ;
      fac[0][tid] = cached ? f16_to_f32(fcs[0][tid]) * a.sl2 : a.sl2;
      fac[2][tid] = cached ? f16_to_f32(fcs[1][tid]) : 1.f;
      if constexpr (FMT == FMT_INT4) {
        fac[1][tid] = cached ? f16_to_f32(fcs[2][tid]) * a.sl2 : 0.f;
        fac[3][tid] = cached ? f16_to_f32(fcs[3][tid]) : 0.f;
      }
    }
  };

  const int prow = perm_key(n);
  const uint32_t k_lane = static_cast<uint32_t>(prow * ROW_BYTES + ((hl ^ (prow & 15)) << 4));
  const int grp16 = lane >> 4, i16 = lane & 15;
  f32x16 o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) o[k] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f, u_run = 0.f;

  auto v_operand = [&](const char *vb, int s) {
    const int ks = s >> 2, blk = s & 3;
    const int row = 16 * ks + 8 * (grp16 >> 1) + (i16 >> 2);
    const int col = 32 * blk + 16 * (grp16 & 1) + 4 * (i16 & 3);
    const bf16x4 lo = __builtin_bit_cast(bf16x4, lds_tr(vb + v_off(row, col >> 3) + 2 * (col & 7)));
    const bf16x4 hi = __builtin_bit_cast(bf16x4, lds_tr(vb + v_off(row + 4, col >> 3) + 2 * (col & 7)));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };

  // One tile from the bf16 tiles: S^T = K Q^T, factors, mask, online softmax,
  // O^T += V^T (P s_v)^T.
  auto compute_tile = [&](int tile, const char *kb, const char *vb, const float (*fac)[64]) {
    const int j0 = (t_lo + tile) * 64;
    uint32_t ka = k_lane;
    asm volatile("" : "+v"(ka));
    f32x16 c0 = f32x16{}, c1 = f32x16{};
    bf16x8 k0 = lds16(kb + ka), k1 = lds16(kb + ka + 32 * ROW_BYTES);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      bf16x8 nk0 = k0, nk1 = k1;
      if (st < 7) {
        const char *kp = kb + (ka ^ ((st + 1) << 5));
        nk0 = lds16(kp);
        nk1 = lds16(kp + 32 * ROW_BYTES);
      }
      __builtin_amdgcn_sched_barrier(0);
      c0 = mfma32(k0, qf[st], c0);
      c1 = mfma32(k1, qf[st], c1);
      k0 = nk0;
      k1 = nk1;
      __builtin_amdgcn_sched_barrier(0);
    }
    // register r of c0 / c1 holds key 16*(r/8) + 8*hl + r%8 (+ 32 for c1)
    auto fac8 = [&](int row, int base) {
      const float4 x = *reinterpret_cast<const float4 *>(&fac[row][base]);
      const float4 y = *reinterpret_cast<const float4 *>(&fac[row][base + 4]);
      return f32x8{x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
    };
    {
      const f32x8 s0a = fac8(0, 8 * hl), s0b = fac8(0, 16 + 8 * hl);
      const f32x8 s1a = fac8(0, 32 + 8 * hl), s1b = fac8(0, 48 + 8 * hl);
      if constexpr (FMT == FMT_INT4) {
        {
          const f32x8 z0a = fac8(1, 8 * hl), z0b = fac8(1, 16 + 8 * hl);
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            c0[r] = fmaf(c0[r], s0a[r], z0a[r] * qsum);
            c0[8 + r] = fmaf(c0[8 + r], s0b[r], z0b[r] * qsum);
          }
        }
        {
          const f32x8 z1a = fac8(1, 32 + 8 * hl), z1b = fac8(1, 48 + 8 * hl);
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            c1[r] = fmaf(c1[r], s1a[r], z1a[r] * qsum);
            c1[8 + r] = fmaf(c1[8 + r], s1b[r], z1b[r] * qsum);
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          c0[r] *= s0a[r];
          c0[8 + r] *= s0b[r];
          c1[r] *= s1a[r];
          c1[8 + r] *= s1b[r];
        }
      }
    }
    if constexpr (LG) {
      if (row_ok) store_logits(a.lg + (static_cast<size_t>(grp) * R + my_row) * a.lg_stride + j0 + 8 * hl, c0, c1);
    }
    if (wave_ragged || j0 + 63 - n_occ > wave_i_min) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ja = j0 + 16 * (r >> 3) + 8 * hl + (r & 7) - n_occ;  // chunk index, < 0 for cache
        c0[r] = (row_ok && ja <= i_q) ? c0[r] : -INFINITY;
        c1[r] = (row_ok && ja + 32 <= i_q) ? c1[r] : -INFINITY;
      }
    }
    float mx = fmaxf(c0[0], c1[0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(c0[r], c1[r]));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (__ballot(mx > m_run + RESCALE_SLACK)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      u_run *= alpha;
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] *= alpha;
      m_run = m_new;
    }
    const float neg_m = (m_run == -INFINITY) ? 0.f : -m_run;
    float ls = 0.f, us = 0.f;
    bf16x8 pb[4];
    {
      const f32x8 v0a = fac8(2, 8 * hl), v0b = fac8(2, 16 + 8 * hl);
      const f32x8 v1a = fac8(2, 32 + 8 * hl), v1b = fac8(2, 48 + 8 * hl);
      f32x8 w0a, w0b, w1a, w1b;
      if constexpr (FMT == FMT_INT4) {
        w0a = fac8(3, 8 * hl);
        w0b = fac8(3, 16 + 8 * hl);
        w1a = fac8(3, 32 + 8 * hl);
        w1b = fac8(3, 48 + 8 * hl);
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float p00 = __builtin_amdgcn_exp2f(c0[r] + neg_m);
        const float p01 = __builtin_amdgcn_exp2f(c0[8 + r] + neg_m);
        const float p10 = __builtin_amdgcn_exp2f(c1[r] + neg_m);
        const float p11 = __builtin_amdgcn_exp2f(c1[8 + r] + neg_m);
        ls += (p00 + p01) + (p10 + p11);
        if constexpr (FMT == FMT_INT4) {
          us = fmaf(p00, w0a[r], us);
          us = fmaf(p01, w0b[r], us);
          us = fmaf(p10, w1a[r], us);
          us = fmaf(p11, w1b[r], us);
        }
        pb[0][r] = static_cast<__bf16>(p00 * v0a[r]);
        pb[1][r] = static_cast<__bf16>(p01 * v0b[r]);
        pb[2][r] = static_cast<__bf16>(p10 * v1a[r]);
        pb[3][r] = static_cast<__bf16>(p11 * v1b[r]);
      }
    }
    l_run += ls;
    u_run += us;
    bf16x8 vc = v_operand(vb, 0);
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      bf16x8 vn = vc;
      if (s < 15) vn = v_operand(vb, s + 1);
      __builtin_amdgcn_sched_barrier(0);
      o[s & 3] = mfma32(vc, pb[s >> 2], o[s & 3]);
      vc = vn;
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if constexpr (NB == 1) {
    // ---- codes one tile ahead in two staging slots; per tile:
    //      [codes(t) landed] barrier, DMA codes(t+1), widen(t), barrier, compute(t)
    char *kb = kbs[0], *vb = vbs[0];
    float (*fac)[64] = facs[0];
    if (ntiles > 0) issue_codes(0, kc0, vc0, fc0);
    for (int t = 0; t < ntiles; t += 2) {
      wait_dma_and_sync();  // codes(t) in slot 0; everyone done with tile t-1
      if (t + 1 < ntiles) issue_codes(t + 1, kc1, vc1, fc1);
      widen_tile(t, kc0, vc0, fc0, kb, vb, fac);
      lds_barrier();
      compute_tile(t, kb, vb, fac);
      if (t + 1 >= ntiles) break;
      wait_dma_and_sync();  // codes(t+1) in slot 1
      if (t + 2 < ntiles) issue_codes(t + 2, kc0, vc0, fc0);
      widen_tile(t + 1, kc1, vc1, fc1, kb, vb, fac);
      lds_barrier();
      compute_tile(t + 1, kb, vb, fac);
    }
  } else {
    // ---- tile t (codes slot and bf16 buffer t & 1), one barrier each:
    //      [widen(t) done, codes(t+1) landed, compute(t-1) done] barrier,
    //      DMA codes(t+2) into the slot widen(t) read, widen(t+1), compute(t)
    if (ntiles > 0) {
      issue_codes(0, kc0, vc0, fc0);
      wait_dma_and_sync();
      if (ntiles > 1) issue_codes(1, kc1, vc1, fc1);
      widen_tile(0, kc0, vc0, fc0, kbs[0], vbs[0], facs[0]);
    }
    for (int t = 0; t < ntiles; t += 2) {
      wait_dma_and_sync();
      if (t + 2 < ntiles) issue_codes(t + 2, kc0, vc0, fc0);
      if (t + 1 < ntiles) widen_tile(t + 1, kc1, vc1, fc1, kbs[1], vbs[1], facs[1]);
      compute_tile(t, kbs[0], vbs[0], facs[0]);
      if (t + 1 >= ntiles) break;
      wait_dma_and_sync();
      if (t + 3 < ntiles) issue_codes(t + 3, kc1, vc1, fc1);
      if (t + 2 < ntiles) widen_tile(t + 2, kc0, vc0, fc0, kbs[0], vbs[0], facs[0]);
      compute_tile(t + 1, kbs[1], vbs[1], facs[1]);
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float u_tot = u_run + __shfl_xor(u_run, 32);
  if (!row_ok) return;
  const size_t li = (static_cast<size_t>(b) * a.Hq + h_q) * a.T + i_q;
  if (a.nsplit > 1) {  // unnormalised partial output and (m, l) of this key split
    const size_t pr = static_cast<size_t>(split) * a.B * a.Hq * a.T + li;
    float *po = a.part + pr * D;
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d = 32 * blk + 8 * a4 + 4 * hl;
        *reinterpret_cast<float4 *>(po + d) = make_float4(o[blk][4 * a4] + u_tot, o[blk][4 * a4 + 1] + u_tot,
                                                          o[blk][4 * a4 + 2] + u_tot, o[blk][4 * a4 + 3] + u_tot);
      }
    }
    if (hl == 0) {
      *reinterpret_cast<float2 *>(a.part_ml + 2 * pr) = make_float2(m_run, l_tot);
      if constexpr (FMT == FMT_INT4) {
        if (split == 0) a.lse2[static_cast<size_t>(a.B) * a.Hq * a.T + li] = qsum;
      }
    }
    return;
  }
  const float inv = 1.f / l_tot;
  uint16_t *orow = static_cast<uint16_t *>(a.out) + li * D;
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int d = 32 * blk + 8 * a4 + 4 * hl;
      *reinterpret_cast<uint2 *>(orow + d) =
          make_uint2(pack_bf16_rne((o[blk][4 * a4] + u_tot) * inv, (o[blk][4 * a4 + 1] + u_tot) * inv),
                     pack_bf16_rne((o[blk][4 * a4 + 2] + u_tot) * inv, (o[blk][4 * a4 + 3] + u_tot) * inv));
    }
  }
  if (hl == 0) {
    const float L = m_run + log2f(l_tot);
    a.lse2[li] = L;
    if (a.lse_nat) a.lse_nat[li] = L * 0.69314718055994530942f;
    if constexpr (FMT == FMT_INT4) a.lse2[static_cast<size_t>(a.B) * a.Hq * a.T + li] = qsum;
  }
}

// ---------------------------------------------------------------------------
// Short chunks (at most 16 packed rows per KV group): the same codes pipeline,
// but each wavefront takes 16 keys of every tile on 16x16 MFMAs, as the native
// short-chunk pass does; the four wavefronts merge at the end.
// ---------------------------------------------------------------------------
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int FMT, bool LG>
__global__ __launch_bounds__(256, 2) void attn_a_qdec(AttnArgs a) {
  using Q = QTile<FMT>;
  // widened bf16 tiles and their per-key factors, double-buffered
  __shared__ __attribute__((aligned(1024))) char kb0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vb0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char kb1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vb1[TILE_BYTES];
  __shared__ __attribute__((aligned(256))) float fac0[4][64];
  __shared__ __attribute__((aligned(256))) float fac1[4][64];
  __shared__ float red_m[4][16], red_l[4][16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g4 = lane >> 4;  // row of the lane; key / d group
  const int R = a.qg * a.T;                 // <= 16
  const int wi_all = xcd_remap(blockIdx.x, gridDim.x);
  const int split = wi_all % a.nsplit;
  const int grp = wi_all / a.nsplit;
  const int g = grp % a.Hkv, b = grp / a.Hkv;
  const bool row_ok = n < R;
  const int i_q = row_ok ? n / a.qg : 0;
  const int h_q = g * a.qg + (row_ok ? n % a.qg : 0);
  const size_t li = (static_cast<size_t>(b) * a.Hq + h_q) * a.T + i_q;
  const int n_occ = a.n_occ;

  bf16x8 qf[4];
  float qsum = 0.f;
  {
    const uint16_t *qrow = static_cast<const uint16_t *>(a.q) + li * D;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row_ok) v = *reinterpret_cast<const uint4 *>(qrow + 32 * st + 8 * g4);
      qf[st] = __builtin_bit_cast(bf16x8, v);
      if constexpr (FMT == FMT_INT4) {
#pragma unroll
        for (int e = 0; e < 8; ++e) qsum += static_cast<float>(qf[st][e]);
      }
    }
    if constexpr (FMT == FMT_INT4) {
      qsum += __shfl_xor(qsum, 16);
      qsum += __shfl_xor(qsum, 32);
      // per-row sum of q for the weight pass of int4 caches (second lse plane)
      if (split == 0 && wave == 0 && g4 == 0 && row_ok)
        a.lse2[static_cast<size_t>(a.B) * a.Hq * a.T + li] = qsum;
    }
  }

  const int key_end = n_occ + (R - 1) / a.qg + 1;
  const int ntiles_all = (key_end + 63) / 64;
  const int per_split = (ntiles_all + a.nsplit - 1) / a.nsplit;
  const int t_lo = split * per_split;
  const int ntiles = min(ntiles_all, t_lo + per_split) - t_lo;
  const size_t cache_row0 = static_cast<size_t>(grp) * a.C;
  const size_t new_row0 = static_cast<size_t>(grp) * a.T;
  // Codes move HBM -> registers with plain vector loads, PD tiles ahead of
  // their use: thread tid holds the 32 codes of key row tid / 4, quarter
  // tid % 4, of K and of V (int8: 2 x 16 bytes each, int4: 16 bytes), and
  // lane l < 16 of wavefront w the fp16 factors of key 16w + l.  Loads into
  // registers keep their order in the vector-memory counter, so each tile
  // waits only for its own loads; an LDS-DMA pipeline this deep would wait
  // for all.  Wavefront w widens, stores and reads back only the rows of its
  // own keys 16w .. 16w + 15, so the wavefronts never wait for each other
  // inside the tile loop.
  constexpr int CW = Q::CODE_ROW / 4 / 16;  // 16-byte words of one thread's share
  constexpr int PD = (FMT == FMT_INT8) ? 2 : 3;
  struct Codes {
    uint4 k[CW], v[CW];
    uint16_t f[Q::NFAC];
  };
  const uint16_t *fsrc[4] = {a.ks, a.vs, a.kz, a.vz};
  const int crow = tid >> 2, cq = tid & 3;   // crow = 16 * wave + lane / 4
  const int fkey = 16 * wave + (lane & 15);  // key of the factors lane < 16 holds
  // Tiles 0 .. nfull-1 of the split lie wholly in the cache: their loads
  // are unconditional, so the compiler can count them (a tile past nfull
  // reloads tile nfull - 1, an L2 hit; every lane loads the factors of key
  // fkey).  The rest (the tile that straddles n_occ, chunk rows)
  // take a direct path after the main loop.
  const int nfull = max(0, min(ntiles, n_occ / 64 - t_lo));
  auto load_codes = [&](int tile, Codes &c) {
    const int j0 = (t_lo + (tile < nfull ? tile : nfull - 1)) * 64;
    const size_t off = (cache_row0 + j0 + crow) * Q::CODE_ROW + cq * (Q::CODE_ROW / 4);
#pragma unroll
    for (int w = 0; w < CW; ++w) {
      c.k[w] = *reinterpret_cast<const uint4 *>(static_cast<const char *>(a.kc) + off + 16 * w);
      c.v[w] = *reinterpret_cast<const uint4 *>(static_cast<const char *>(a.vc) + off + 16 * w);
    }
#pragma unroll
    for (int f = 0; f < Q::NFAC; ++f) c.f[f] = fsrc[f][cache_row0 + j0 + fkey];
  };
  auto store = [&](char *kb, char *vb, const uint4 (&kw)[4], const uint4 (&vw)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<uint4 *>(kb + kq_off(crow, 4 * cq + i)) = kw[i];
      *reinterpret_cast<uint4 *>(vb + v_off(crow, 4 * cq + i)) = vw[i];
    }
  };
  auto store_fac = [&](float (*fac)[64], bool cached, const uint16_t *f) {
    fac[0][fkey] = cached ? f16_to_f32(f[0]) * a.sl2 : a.sl2;
    fac[2][fkey] = cached ? f16_to_f32(f[1]) : 1.f;
    if constexpr (FMT == FMT_INT4) {
      fac[1][fkey] = cached ? f16_to_f32(f[2]) * a.sl2 : 0.f;
      fac[3][fkey] = cached ? f16_to_f32(f[3]) : 0.f;
    }
  };
  // a tile wholly in the cache, from the prefetched registers
  auto widen_full = [&](const Codes &c, char *kb, char *vb, float (*fac)[64]) {
    uint4 kw[4], vw[4];
    widen32<FMT>(reinterpret_cast<const char *>(c.k), kw);
    widen32<FMT>(reinterpret_cast<const char *>(c.v), vw);
    store(kb, vb, kw, vw);
    if (lane < 16) store_fac(fac, true, c.f);
  };
  // any other tile, loading as it goes: codes of rows below n_occ, new keys
  // (bf16) above, zeros past the chunk
  auto widen_direct = [&](int tile, char *kb, char *vb, float (*fac)[64]) {
    const int j0 = (t_lo + tile) * 64;
    const int j = j0 + crow;
    uint4 kw[4], vw[4];
    if (j < n_occ) {
      const size_t off = (cache_row0 + j) * Q::CODE_ROW + cq * (Q::CODE_ROW / 4);
      widen32<FMT>(static_cast<const char *>(a.kc) + off, kw);
      widen32<FMT>(static_cast<const char *>(a.vc) + off, vw);
    } else {
      const int t = j - n_occ;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kw[i] = vw[i] = make_uint4(0, 0, 0, 0);
        if (t < a.T) {
          const size_t e = (new_row0 + t) * D + 32 * cq + 8 * i;
          kw[i] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.kn) + e);
          vw[i] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.vn) + e);
        }
      }
    }
    store(kb, vb, kw, vw);
    if (lane < 16) {
      const bool cached = j0 + fkey < n_occ;
      uint16_t f[4] = {0, 0, 0, 0};
      if (cached) {
#pragma unroll
        for (int q = 0; q < Q::NFAC; ++q) f[q] = fsrc[q][cache_row0 + j0 + fkey];
      }
      store_fac(fac, cached, f);
    }
  };

  f32x4 o[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f, u_run = 0.f;
  const int krow = 16 * wave + n;
  const int kk0 = 16 * wave + 4 * g4;  // tile key of the lane's first value

  auto compute = [&](int tile, const char *kb, const char *vb, const float (*fac)[64]) {
    const int j0 = (t_lo + tile) * 64;
    f32x4 c = f32x4{};
#pragma unroll
    for (int st = 0; st < 4; ++st)
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds16(kb + kq_off(krow, 4 * st + g4)), qf[st], c, 0, 0, 0);
    // c[i]: tile key kk0 + i of row n; factors bring it to log2 units
    const float4 s4 = *reinterpret_cast<const float4 *>(&fac[0][kk0]);
    const float sk[4] = {s4.x, s4.y, s4.z, s4.w};
    float zk[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (FMT == FMT_INT4) {
      const float4 z4 = *reinterpret_cast<const float4 *>(&fac[1][kk0]);
      zk[0] = z4.x;
      zk[1] = z4.y;
      zk[2] = z4.z;
      zk[3] = z4.w;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = (FMT == FMT_INT4) ? fmaf(c[i], sk[i], zk[i] * qsum) : c[i] * sk[i];
    if constexpr (LG) {
      if (row_ok)
        *reinterpret_cast<float4 *>(a.lg + (static_cast<size_t>(grp) * R + n) * a.lg_stride + j0 + kk0) =
            make_float4(c[0], c[1], c[2], c[3]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ja = j0 + kk0 + i - n_occ;
      c[i] = (row_ok && ja <= i_q) ? c[i] : -INFINITY;
    }
    float mx = fmaxf(fmaxf(c[0], c[1]), fmaxf(c[2], c[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (mx > m_run + RESCALE_SLACK) {
      const float alpha = (m_run == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - mx);
      l_run *= alpha;
      u_run *= alpha;
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] *= alpha;
      m_run = mx;
    }
    const float neg_m = (m_run == -INFINITY) ? 0.f : -m_run;
    const float4 v4 = *reinterpret_cast<const float4 *>(&fac[2][kk0]);
    const float sv[4] = {v4.x, v4.y, v4.z, v4.w};
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(c[i] + neg_m);
    l_run += (p[0] + p[1]) + (p[2] + p[3]);
    if constexpr (FMT == FMT_INT4) {
      const float4 w4 = *reinterpret_cast<const float4 *>(&fac[3][kk0]);
      u_run = fmaf(p[0], w4.x, fmaf(p[1], w4.y, fmaf(p[2], w4.z, fmaf(p[3], w4.w, u_run))));
    }
    const i16x4 pb = __builtin_bit_cast(
        i16x4, make_uint2(pack_bf16_rne(p[0] * sv[0], p[1] * sv[1]), pack_bf16_rne(p[2] * sv[2], p[3] * sv[3])));
    const int vrow = 16 * wave + 4 * g4 + (n >> 2);
#pragma unroll
    for (int dblk = 0; dblk < 8; ++dblk) {
      const int col = 16 * dblk + 4 * (n & 3);
      const i16x4 va = lds_tr(vb + v_off(vrow, col >> 3) + 2 * (col & 7));
      o[dblk] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, o[dblk], 0, 0, 0);
    }
  };

  // Tile t: widen into buffer t & 1, refill its registers with tile t + PD,
  // compute.  Lanes read rows that other lanes of their wavefront wrote;
  // wave_lds_sync keeps the reads of tile t after its writes, and (one tile
  // on) the reads of tile t - 1 before the writes of tile t + 1 into the
  // same buffer.
  // Groups of G tiles are unrolled straight-line: the compiler counts the
  // loads in flight exactly there, while across a loop back-edge it waits
  // for all of them (so it drains once per group, not once per tile).
  if (nfull > 0) {
    constexpr int G = 3 * PD;
    Codes cr[PD];
#pragma unroll
    for (int p = 0; p < PD; ++p) load_codes(p, cr[p]);
    for (int t0 = 0; t0 < nfull; t0 += G) {
#pragma unroll
      for (int p = 0; p < G; ++p) {
        const int t = t0 + p;
        char *kb = (p & 1) ? kb1 : kb0;  // t0 is even: t & 1 == p & 1
        char *vb = (p & 1) ? vb1 : vb0;
        float (*fac)[64] = (p & 1) ? fac1 : fac0;
        if (t < nfull) widen_full(cr[p % PD], kb, vb, fac);
        load_codes(t + PD, cr[p % PD]);
        if (t < nfull) {
          wave_lds_sync();
          compute(t, kb, vb, fac);
        }
      }
    }
  }
  for (int t = nfull; t < ntiles; ++t) {
    char *kb = (t & 1) ? kb1 : kb0;
    char *vb = (t & 1) ? vb1 : vb0;
    float (*fac)[64] = (t & 1) ? fac1 : fac0;
    widen_direct(t, kb, vb, fac);
    wave_lds_sync();
    compute(t, kb, vb, fac);
  }

  // ---- merge the four wavefronts (u: the zero-point term, the same for every d) ----
  float l_w = l_run + __shfl_xor(l_run, 16);
  l_w += __shfl_xor(l_w, 32);
  float u_w = u_run + __shfl_xor(u_run, 16);
  u_w += __shfl_xor(u_w, 32);
  if (g4 == 0) {
    red_m[wave][n] = m_run;
    red_l[wave][n] = l_w;
  }
  __syncthreads();  // also: every wavefront is done with the tiles
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, red_m[w][n]);
  const float my_scale = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
  auto red_o = [&](int w) { return reinterpret_cast<float *>(w < 2 ? kb0 : vb0) + (w & 1) * 16 * D; };
  {
    float *mine = red_o(wave);
#pragma unroll
    for (int dblk = 0; dblk < 8; ++dblk)
      *reinterpret_cast<float4 *>(mine + n * D + 16 * dblk + 4 * g4) =
          make_float4((o[dblk][0] + u_w) * my_scale, (o[dblk][1] + u_w) * my_scale,
                      (o[dblk][2] + u_w) * my_scale, (o[dblk][3] + u_w) * my_scale);
  }
  __syncthreads();
  const int rr = tid >> 4, d0 = 8 * (tid & 15);
  if (rr >= R) return;
  const int ri = rr / a.qg, rh = g * a.qg + rr % a.qg;
  const size_t lr = (static_cast<size_t>(b) * a.Hq + rh) * a.T + ri;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
#pragma unroll
    for (int e4 = 0; e4 < 2; ++e4) {
      const float4 v = *reinterpret_cast<const float4 *>(red_o(w) + rr * D + d0 + 4 * e4);
      acc[4 * e4] += v.x;
      acc[4 * e4 + 1] += v.y;
      acc[4 * e4 + 2] += v.z;
      acc[4 * e4 + 3] += v.w;
    }
  }
  float Mr = -INFINITY, lr_tot = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) Mr = fmaxf(Mr, red_m[w][rr]);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float mw = red_m[w][rr];
    lr_tot += (mw == -INFINITY) ? 0.f : red_l[w][rr] * __builtin_amdgcn_exp2f(mw - Mr);
  }
  const size_t plane = static_cast<size_t>(a.B) * a.Hq * a.T;
  if (a.nsplit > 1) {
    const size_t pr = static_cast<size_t>(split) * plane + lr;
    float *po = a.part + pr * D + d0;
    *reinterpret_cast<float4 *>(po) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    *reinterpret_cast<float4 *>(po + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    if (d0 == 0) *reinterpret_cast<float2 *>(a.part_ml + 2 * pr) = make_float2(Mr, lr_tot);
    return;
  }
  const float inv = 1.f / lr_tot;
  uint16_t *orow = static_cast<uint16_t *>(a.out) + lr * D + d0;
  *reinterpret_cast<uint4 *>(orow) =
      make_uint4(pack_bf16_rne(acc[0] * inv, acc[1] * inv), pack_bf16_rne(acc[2] * inv, acc[3] * inv),
                 pack_bf16_rne(acc[4] * inv, acc[5] * inv), pack_bf16_rne(acc[6] * inv, acc[7] * inv));
  if (d0 == 0) {
    const float L = Mr + log2f(lr_tot);
    a.lse2[lr] = L;
    if (a.lse_nat) a.lse_nat[lr] = L * 0.69314718055994530942f;
  }
}

}  // namespace

hipError_t launch_attn_a_quant_d128(const AttnArgs &a, hipStream_t s) {
  const int groups = a.B * a.Hkv;
  const int R = a.qg * a.T;
  const int nA = groups * ((R + 127) / 128) * a.nsplit;
  KernelTimer timer(H2O_K_ATTN_A, s);
  if (R <= 16) {  // short chunks: 16 keys of each tile per wavefront
    const int nD = groups * a.nsplit;
    if (a.cache_fmt == FMT_INT8) {
      if (a.lg) {
        hipLaunchKernelGGL((attn_a_qdec<FMT_INT8, true>), dim3(nD), dim3(256), 0, s, a);
      } else {
        hipLaunchKernelGGL((attn_a_qdec<FMT_INT8, false>), dim3(nD), dim3(256), 0, s, a);
      }
    } else if (a.lg) {
      hipLaunchKernelGGL((attn_a_qdec<FMT_INT4, true>), dim3(nD), dim3(256), 0, s, a);
    } else {
      hipLaunchKernelGGL((attn_a_qdec<FMT_INT4, false>), dim3(nD), dim3(256), 0, s, a);
    }
    return hipGetLastError();
  }
  auto launch_long = [&](auto fmt_tag) {
    constexpr int FMT = decltype(fmt_tag)::value;
    if (a.lg) {
      hipLaunchKernelGGL((attn_a_quant<FMT, true, 4>), dim3(nA), dim3(256), 0, s, a);
    } else if (R >= 256) {  // long chunks: 256 rows per block share each widened tile
      const int n8 = groups * ((R + 255) / 256) * a.nsplit;
      hipLaunchKernelGGL((attn_a_quant<FMT, false, 8>), dim3(n8), dim3(512), 0, s, a);
    } else {
      hipLaunchKernelGGL((attn_a_quant<FMT, false, 4>), dim3(nA), dim3(256), 0, s, a);
    }
  };
  if (a.cache_fmt == FMT_INT8) {
    launch_long(std::integral_constant<int, FMT_INT8>{});
  } else {
    launch_long(std::integral_constant<int, FMT_INT4>{});
  }
  return hipGetLastError();
}

}  // namespace h2o
