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
// OFF16 (4-bit keys): code n widens to 16 + n, see below.  8-bit codes: the
// second 16 bytes at `hi` (default codes + 16).
template <int FMT, bool OFF16 = false>
__device__ __forceinline__ void widen32(const char *codes, uint4 (&out)[4], const char *hi = nullptr) {
  if constexpr (FMT == FMT_INT8) {
    const uint4 a = *reinterpret_cast<const uint4 *>(codes);
    const uint4 b = *reinterpret_cast<const uint4 *>(hi ? hi : codes + 16);
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
  } else if constexpr (OFF16) {
    // A 4-bit key code n widens to 16 + n, whose bf16 pattern is
    // 0x4180 | n << 3 (exponent of 16, n in the top 4 of the 7 mantissa
    // bits): no conversion instruction, and 16 + n is still an integer exact
    // in bf16.  The logits take the offset back out through the zero point:
    // s n + z = s (16 + n) + (z - 16 s).  (Values keep their codes: there
    // the offset would pass through the bf16-rounded P s_v and cost accuracy.)
    const uint4 a = *reinterpret_cast<const uint4 *>(codes);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // even elements are the low nibbles, odd ones the high nibbles
      const uint32_t ev = w[i] & 0x0f0f0f0fu, od = (w[i] >> 4) & 0x0f0f0f0fu;
      uint32_t r[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // bytes [ev_q, 0, od_q, 0] (selector 0x0c yields a zero byte)
        const uint32_t sel = 0x0c000c00u | ((4u + q) << 16) | static_cast<uint32_t>(q);
        const uint32_t y = __builtin_amdgcn_perm(od, ev, sel);
        r[q] = (y << 3) | 0x41804180u;
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
  int t_lo, ntiles;  // key tiles t_lo .. t_lo + ntiles - 1 of this split (ntiles 0: none)
  split_tiles(ntiles_all, a.nsplit, split, t_lo, ntiles);
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
      uint32_t off = static_cast<uint32_t>(sgm * 1024 + 16 * lane);
      if constexpr (FMT == FMT_INT8) {  // 16-byte chunk c of code row r lands at c ^ ((r >> 1) & 1)
        const int row = sgm * 8 + (lane >> 3);
        off = static_cast<uint32_t>(row * Q::CODE_ROW + 16 * ((lane & 7) ^ ((row >> 1) & 1)));
      }
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
  // 8-bit code rows sit in the staging slot with 16-byte chunk c at position
  // c ^ ((r >> 1) & 1): the 4 rows x 4 quarters that 16 lanes read at once
  // then meet 16 distinct bank groups (in order, rows r and r + 2 met the
  // same 8); 4-bit rows (64 bytes) already do.
  auto widen_rows = [&](int j, const char *cs, const void *nsrc, char *dst, bool is_v) {
    uint4 w[4];
    if (j < n_occ) {
      const char *row = cs + crow * Q::CODE_ROW;
      const char *lo = row + cq * (Q::CODE_ROW / 4), *hi = nullptr;
      if constexpr (FMT == FMT_INT8) {
        const int sw = (crow >> 1) & 1;
        lo = row + 16 * ((2 * cq) ^ sw);
        hi = row + 16 * ((2 * cq + 1) ^ sw);
      }
      if (is_v) {
        widen32<FMT>(lo, w, hi);
      } else {
        widen32<FMT, true>(lo, w, hi);
      }
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
      *reinterpret_cast<uint4 *>(dst + (is_v ? vq_off(crow, 4 * cq + i) : kq_off(crow, 4 * cq + i))) = w[i];
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
        // the widened key codes are 16 + n: k = s n + z = s (16 + n) + (z - 16 s)
        fac[1][tid] = cached ? (f16_to_f32(fcs[2][tid]) - 16.f * f16_to_f32(fcs[0][tid])) * a.sl2 : 0.f;
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
    const bf16x4 lo = __builtin_bit_cast(bf16x4, lds_tr(vb + vq_off(row, col >> 3) + 2 * (col & 7)));
    const bf16x4 hi = __builtin_bit_cast(bf16x4, lds_tr(vb + vq_off(row + 4, col >> 3) + 2 * (col & 7)));
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
    float mx = __builtin_fmaxf(__builtin_fmaxf(c0[0], c1[0]), c0[1]);
#pragma unroll
    for (int r = 1; r < 15; ++r) mx = __builtin_fmaxf(__builtin_fmaxf(mx, c1[r]), c0[r + 1]);
    mx = __builtin_fmaxf(mx, c1[15]);
    mx = max_xor32(mx);  // the other half-wave holds the other 32 keys of the lane's row
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
// Short chunks (at most 16 packed rows per KV group).  Each wavefront takes
// 16 keys of every 64-key tile of its split on 16x16 MFMAs, and the four
// wavefronts merge at the end.  The codes go HBM -> registers with plain
// loads, NPF tiles ahead, and widen in registers straight into the MFMA
// operands: nothing passes through LDS between load and use, and no
// wavefront waits for another inside the tile loop.  The pace is set by the
// per-tile instruction chain (widening, products, softmax), not by the loads:
// with the loads taken out the pass is about as slow, and rings deeper than
// two tiles or eight wavefronts per block measured slower.
//
// Head-dimension order inside the products.  One permutation of d applied
// to both operands of S = K Q^T leaves every dot product unchanged, and one
// applied to V's columns only relabels O's; both are chosen so that a lane's
// share of an operand is contiguous in a code row:
//   S (steps st = 0..3 of 16x16x32): lane (n, g) = (lane % 16, lane / 16)
//     supplies key n and query row n at d = 32 g + 8 st + e, e = 0..7;
//   O^T += V^T P^T (blocks k = 0..7 of 16x16x16): lane (m, g) supplies
//     d = 8 m + k of keys 4 g + i, i = 0..3 (bytes 8m.. of an 8-bit code row,
//     4m.. of a 4-bit one); its accumulator register i of block k then holds
//     d = 32 g + 8 i + k of query row lane % 16.
// ---------------------------------------------------------------------------
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// bf16 patterns of two fp32 values that bf16 holds exactly, as one word
__device__ __forceinline__ uint32_t hi16_pair(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// 8 consecutive codes of a row (8-bit: 8 bytes; 4-bit: 4 bytes, low nibble
// first) -> 8 bf16, as they are (no offset).
template <int FMT>
__device__ __forceinline__ uint4 widen8(const char *p) {
  if constexpr (FMT == FMT_INT8) {
    const uint2 x = *reinterpret_cast<const uint2 *>(p);
    const int32_t w[2] = {static_cast<int32_t>(x.x), static_cast<int32_t>(x.y)};
    uint32_t r[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      r[2 * h] = hi16_pair(static_cast<float>((w[h] << 24) >> 24), static_cast<float>((w[h] << 16) >> 24));
      r[2 * h + 1] = hi16_pair(static_cast<float>((w[h] << 8) >> 24), static_cast<float>(w[h] >> 24));
    }
    return make_uint4(r[0], r[1], r[2], r[3]);
  } else {
    const uint32_t x = *reinterpret_cast<const uint32_t *>(p);
    uint32_t r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      r[q] = hi16_pair(static_cast<float>((x >> (8 * q)) & 15u), static_cast<float>((x >> (8 * q + 4)) & 15u));
    return make_uint4(r[0], r[1], r[2], r[3]);
  }
}

// One lane's share of one tile wholly in the cache, as loaded.
template <int FMT>
struct DecShare {
  static constexpr int KW = FMT == FMT_INT8 ? 2 : 1;  // 16-byte words of key codes (key n)
  static constexpr int VW = FMT == FMT_INT8 ? 8 : 4;  // 32-bit words of value codes (keys 4g + i)
  static constexpr int NF = FMT == FMT_INT8 ? 2 : 4;  // factor arrays: ks, vs (, kz, vz)
  uint4 k[KW];
  uint32_t v[VW];
  uint2 f[NF];  // fp16 factors of keys 4g .. 4g + 3
};

template <int FMT, bool LG, int NPF, int NW>
__global__ __launch_bounds__(64 * NW, NW / 2) void attn_a_qdec(AttnArgs a) {
  using Sh = DecShare<FMT>;
  constexpr int CODE_ROW = QTile<FMT>::CODE_ROW;
  constexpr int RS = D + 4;  // row stride of the merge rows (floats): 16 rows meet distinct banks
  __shared__ __attribute__((aligned(16))) float red_o[NW][16 * RS];
  __shared__ float red_m[NW][16], red_l[NW][16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g4 = lane >> 4;  // row / key of the lane; key / d group
  // wavefront w takes keys 16 (w % 4) .. + 15 of the tiles t = tpar (mod TS)
  constexpr int TS = NW / 4;
  const int wq = wave & 3, tpar = wave >> 2;
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

  bf16x8 qf[4];  // step st: d = 32 g4 + 8 st .. + 7 of row n
  float qsum = 0.f;
  {
    const uint16_t *qrow = static_cast<const uint16_t *>(a.q) + li * D + 32 * g4;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row_ok) v = *reinterpret_cast<const uint4 *>(qrow + 8 * st);
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
  int t_lo, ntiles;  // key tiles t_lo .. t_lo + ntiles - 1 of this split (ntiles 0: none)
  split_tiles(ntiles_all, a.nsplit, split, t_lo, ntiles);
  const size_t cache_row0 = static_cast<size_t>(grp) * a.C;
  const size_t new_row0 = static_cast<size_t>(grp) * a.T;
  const char *kcb = static_cast<const char *>(a.kc), *vcb = static_cast<const char *>(a.vc);
  const uint16_t *fsrc[4] = {a.ks, a.vs, a.kz, a.vz};
  const int kk0 = 16 * wq + 4 * g4;  // tile key of the lane's first logit

  // Tiles 0 .. nfull-1 of the split lie wholly in the cache and take the
  // prefetched path; the rest (the tile that straddles n_occ, chunk keys)
  // load as they go.
  const int nfull = max(0, min(ntiles, n_occ / 64 - t_lo));
  auto load_share = [&](int tile, Sh &s) {
    const size_t jw = cache_row0 + static_cast<size_t>(t_lo + tile) * 64 + 16 * wq;
    const char *kp = kcb + (jw + n) * CODE_ROW + g4 * (CODE_ROW / 4);
#pragma unroll
    for (int w = 0; w < Sh::KW; ++w) s.k[w] = *reinterpret_cast<const uint4 *>(kp + 16 * w);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const char *vp = vcb + (jw + 4 * g4 + i) * CODE_ROW + n * (CODE_ROW / 16);
      if constexpr (FMT == FMT_INT8) {
        const uint2 x = *reinterpret_cast<const uint2 *>(vp);
        s.v[2 * i] = x.x;
        s.v[2 * i + 1] = x.y;
      } else {
        s.v[i] = *reinterpret_cast<const uint32_t *>(vp);
      }
    }
#pragma unroll
    for (int f = 0; f < Sh::NF; ++f) __builtin_memcpy(&s.f[f], fsrc[f] + jw + 4 * g4, sizeof(uint2));
  };

  f32x4 o[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f, u_run = 0.f;

  // One tile: kw the lane's K operands (bf16), sk / zk / sv / zv the factors
  // of keys kk0 + i, vop(k) the lane's V operand of block k.
  // masked false (tiles wholly below n_occ): every key is visible to every
  // row, and rows past R compute values that are never written.
  auto tile_body = [&](int tile, const uint4 (&kw)[4], const float (&sk)[4], const float (&zk)[4],
                       const float (&sv)[4], const float (&zv)[4], auto &&vop, auto masked) {
    const int j0 = (t_lo + tile) * 64;
    f32x4 c = f32x4{};
#pragma unroll
    for (int st = 0; st < 4; ++st)
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kw[st]), qf[st], c, 0, 0, 0);
    // c[i]: tile key kk0 + i of row n; factors bring it to log2 units
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = (FMT == FMT_INT4) ? fmaf(c[i], sk[i], zk[i] * qsum) : c[i] * sk[i];
    if constexpr (LG) {
      if (row_ok)
        *reinterpret_cast<float4 *>(a.lg + (static_cast<size_t>(grp) * R + n) * a.lg_stride + j0 + kk0) =
            make_float4(c[0], c[1], c[2], c[3]);
    }
    if constexpr (decltype(masked)::value) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ja = j0 + kk0 + i - n_occ;
        c[i] = (row_ok && ja <= i_q) ? c[i] : -INFINITY;
      }
    }
    float mx = __builtin_fmaxf(__builtin_fmaxf(c[0], c[1]), __builtin_fmaxf(c[2], c[3]));
    mx = max_xor32(max_xor16(mx));
    if (mx > m_run + RESCALE_SLACK) {
      const float alpha = (m_run == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - mx);
      l_run *= alpha;
      u_run *= alpha;
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] *= alpha;
      m_run = mx;
    }
    const float neg_m = (m_run == -INFINITY) ? 0.f : -m_run;
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(c[i] + neg_m);
    l_run += (p[0] + p[1]) + (p[2] + p[3]);
    if constexpr (FMT == FMT_INT4) u_run = fmaf(p[0], zv[0], fmaf(p[1], zv[1], fmaf(p[2], zv[2], fmaf(p[3], zv[3], u_run))));
    const i16x4 pb = __builtin_bit_cast(
        i16x4, make_uint2(pack_bf16_hw(p[0] * sv[0], p[1] * sv[1]), pack_bf16_hw(p[2] * sv[2], p[3] * sv[3])));
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop(k), pb, o[k], 0, 0, 0);
  };

  // a tile wholly in the cache, from its loaded share
  auto full_tile = [&](int tile, const Sh &s) {
    uint4 kw[4];
    widen32<FMT, FMT == FMT_INT4>(reinterpret_cast<const char *>(s.k), kw);
    float sk[4], zk[4], sv[4], zv[4];
    const f16x4 fks = __builtin_bit_cast(f16x4, s.f[0]), fvs = __builtin_bit_cast(f16x4, s.f[1]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sk[i] = static_cast<float>(fks[i]) * a.sl2;
      sv[i] = static_cast<float>(fvs[i]);
      zk[i] = zv[i] = 0.f;
    }
    if constexpr (FMT == FMT_INT4) {
      // the widened key codes are 16 + n: k = s n + z = s (16 + n) + (z - 16 s)
      const f16x4 fkz = __builtin_bit_cast(f16x4, s.f[2]), fvz = __builtin_bit_cast(f16x4, s.f[3]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        zk[i] = (static_cast<float>(fkz[i]) - 16.f * static_cast<float>(fks[i])) * a.sl2;
        zv[i] = static_cast<float>(fvz[i]);
      }
    }
    if constexpr (FMT == FMT_INT8) {
      tile_body(tile, kw, sk, zk, sv, zv, [&](int k) {
        float f[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int32_t w = static_cast<int32_t>(s.v[2 * i + (k >> 2)]);
          f[i] = static_cast<float>((w << (24 - 8 * (k & 3))) >> 24);
        }
        return __builtin_bit_cast(i16x4, make_uint2(hi16_pair(f[0], f[1]), hi16_pair(f[2], f[3])));
      }, std::false_type{});
    } else {
      uint32_t nib[4];  // the lane's nibble k of row i sits in byte k / 2 of nib[i] (>> 4 if k odd)
#pragma unroll
      for (int i = 0; i < 4; ++i) nib[i] = s.v[i];
      tile_body(tile, kw, sk, zk, sv, zv, [&](int k) {
        float f[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t x = (k & 1) ? ((nib[i] >> 4) & 0x0f0f0f0fu) : (nib[i] & 0x0f0f0f0fu);
          f[i] = static_cast<float>((x >> (8 * (k >> 1))) & 0xffu);
        }
        return __builtin_bit_cast(i16x4, make_uint2(hi16_pair(f[0], f[1]), hi16_pair(f[2], f[3])));
      }, std::false_type{});
    }
  };

  // any other tile: codes of rows below n_occ, new keys (bf16) above, zeros
  // past the chunk
  auto tail_tile = [&](int tile) {
    const int j0 = (t_lo + tile) * 64;
    const int jk = j0 + 16 * wq + n;  // key row of the lane's K operand
    uint4 kw[4];
    if (jk < n_occ) {
      widen32<FMT, FMT == FMT_INT4>(kcb + (cache_row0 + jk) * CODE_ROW + g4 * (CODE_ROW / 4), kw);
    } else {
      const int t = jk - n_occ;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        kw[st] = make_uint4(0, 0, 0, 0);
        if (t < a.T)
          kw[st] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.kn) + (new_row0 + t) * D +
                                                    32 * g4 + 8 * st);
      }
    }
    uint4 vrow[4];  // d = 8n .. 8n + 7 of key kk0 + i, bf16
    float sk[4], zk[4], sv[4], zv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j0 + kk0 + i;
      if (j < n_occ) {
        const size_t row = cache_row0 + j;
        vrow[i] = widen8<FMT>(vcb + row * CODE_ROW + n * (CODE_ROW / 16));
        const float s_k = f16_to_f32(a.ks[row]);
        sk[i] = s_k * a.sl2;
        sv[i] = f16_to_f32(a.vs[row]);
        zk[i] = zv[i] = 0.f;
        if constexpr (FMT == FMT_INT4) {
          zk[i] = (f16_to_f32(a.kz[row]) - 16.f * s_k) * a.sl2;
          zv[i] = f16_to_f32(a.vz[row]);
        }
      } else {
        const int t = j - n_occ;
        vrow[i] = make_uint4(0, 0, 0, 0);
        if (t < a.T)
          vrow[i] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.vn) + (new_row0 + t) * D + 8 * n);
        sk[i] = a.sl2;
        sv[i] = 1.f;
        zk[i] = zv[i] = 0.f;
      }
    }
    tile_body(tile, kw, sk, zk, sv, zv, [&](int k) {
      auto el = [&](const uint4 &r) {
        const uint32_t w = (k >> 1) == 0 ? r.x : (k >> 1) == 1 ? r.y : (k >> 1) == 2 ? r.z : r.w;
        return (k & 1) ? (w >> 16) : (w & 0xffffu);
      };
      return __builtin_bit_cast(i16x4, make_uint2(el(vrow[0]) | (el(vrow[1]) << 16), el(vrow[2]) | (el(vrow[3]) << 16)));
    }, std::true_type{});
  };

  // Full tiles through a ring of NPF shares: the share of the wavefront's
  // u-th tile is loaded NPF of its tiles before its use.  Inside the loop
  // every load is unconditional, so the compiler counts the loads in flight
  // exactly.
  const int mfull = nfull > tpar ? (nfull - tpar + TS - 1) / TS : 0;    // the wavefront's full tiles
  const int mtiles = ntiles > tpar ? (ntiles - tpar + TS - 1) / TS : 0;  // and all its tiles
  if (mfull > 0) {
    Sh sh[NPF];
#pragma unroll
    for (int p = 0; p < NPF; ++p) load_share(min(p, mfull - 1) * TS + tpar, sh[p]);
    int u = 0;
    for (; u + 2 * NPF <= mfull; u += NPF) {
#pragma unroll
      for (int p = 0; p < NPF; ++p) {
        full_tile((u + p) * TS + tpar, sh[p]);
        load_share((u + p + NPF) * TS + tpar, sh[p]);
      }
    }
    // fewer than 2 NPF full tiles left, the first NPF of them (or all) loaded
#pragma unroll
    for (int p = 0; p < NPF; ++p) {
      if (u + p < mfull) {
        full_tile((u + p) * TS + tpar, sh[p]);
        if (u + p + NPF < mfull) load_share((u + p + NPF) * TS + tpar, sh[p]);
      }
    }
#pragma unroll
    for (int p = 0; p < NPF; ++p)
      if (u + NPF + p < mfull) full_tile((u + NPF + p) * TS + tpar, sh[p]);
  }
  for (int u = mfull; u < mtiles; ++u) tail_tile(u * TS + tpar);

  // ---- merge the four wavefronts (u: the zero-point term, the same for every d) ----
  float l_w = l_run + __shfl_xor(l_run, 16);
  l_w += __shfl_xor(l_w, 32);
  float u_w = u_run + __shfl_xor(u_run, 16);
  u_w += __shfl_xor(u_w, 32);
  if (g4 == 0) {
    red_m[wave][n] = m_run;
    red_l[wave][n] = l_w;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) M = fmaxf(M, red_m[w][n]);
  const float my_scale = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
  {
    float *mine = red_o[wave] + n * RS + 32 * g4;  // d = 32 g4 + 8 i + k at mine[8 i + k]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<float4 *>(mine + 8 * i) =
          make_float4((o[0][i] + u_w) * my_scale, (o[1][i] + u_w) * my_scale, (o[2][i] + u_w) * my_scale,
                      (o[3][i] + u_w) * my_scale);
      *reinterpret_cast<float4 *>(mine + 8 * i + 4) =
          make_float4((o[4][i] + u_w) * my_scale, (o[5][i] + u_w) * my_scale, (o[6][i] + u_w) * my_scale,
                      (o[7][i] + u_w) * my_scale);
    }
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
  for (int w = 0; w < NW; ++w) {
#pragma unroll
    for (int e4 = 0; e4 < 2; ++e4) {
      const float4 v = *reinterpret_cast<const float4 *>(red_o[w] + rr * RS + d0 + 4 * e4);
      acc[4 * e4] += v.x;
      acc[4 * e4 + 1] += v.y;
      acc[4 * e4 + 2] += v.z;
      acc[4 * e4 + 3] += v.w;
    }
  }
  float Mr = -INFINITY, lr_tot = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) Mr = fmaxf(Mr, red_m[w][rr]);
#pragma unroll
  for (int w = 0; w < NW; ++w) {
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
    // tiles each wavefront keeps in flight (4 KB of 8-bit / 2 KB of 4-bit
    // codes each) and wavefronts per block
    constexpr int PF8 = 2, PF4 = 2, NWD = 4;
    const int nD = groups * a.nsplit;
    if (a.cache_fmt == FMT_INT8) {
      if (a.lg) {
        hipLaunchKernelGGL((attn_a_qdec<FMT_INT8, true, PF8, NWD>), dim3(nD), dim3(64 * NWD), 0, s, a);
      } else {
        hipLaunchKernelGGL((attn_a_qdec<FMT_INT8, false, PF8, NWD>), dim3(nD), dim3(64 * NWD), 0, s, a);
      }
    } else if (a.lg) {
      hipLaunchKernelGGL((attn_a_qdec<FMT_INT4, true, PF4, NWD>), dim3(nD), dim3(64 * NWD), 0, s, a);
    } else {
      hipLaunchKernelGGL((attn_a_qdec<FMT_INT4, false, PF4, NWD>), dim3(nD), dim3(64 * NWD), 0, s, a);
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
