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
#include "code_widen.hpp"
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

// NW: wavefronts per block (4 or 8), 32 rows each; a widened tile serves them all.
template <int FMT, int NW>
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
  // mid() runs right after the S MFMAs are issued: with 8 wavefronts it widens
  // the next tile, whose vector and LDS work then overlaps this tile's matrix
  // work (before, every wavefront widened first and then computed, so the two
  // wavefronts of a SIMD were in the same phase at once).
  auto compute_tile = [&](int tile, const char *kb, const char *vb, const float (*fac)[64], auto &&mid) {
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
    mid();
    __builtin_amdgcn_sched_barrier(0);
    // register r of c0 / c1 holds key 16*(r/8) + 8*hl + r%8 (+ 32 for c1)
    auto fac8 = [&](int row, int base) {
      const float4 x = *reinterpret_cast<const float4 *>(&fac[row][base]);
      const float4 y = *reinterpret_cast<const float4 *>(&fac[row][base + 4]);
      return f32x8{x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
    };
    // The logits in log2 units relative to the running maximum, which the
    // factor FMA subtracts (m_run = -inf: the logits themselves).
    const float neg_m = (m_run == -INFINITY) ? 0.f : -m_run;
    {
      const f32x8 s0a = fac8(0, 8 * hl), s0b = fac8(0, 16 + 8 * hl);
      const f32x8 s1a = fac8(0, 32 + 8 * hl), s1b = fac8(0, 48 + 8 * hl);
      if constexpr (FMT == FMT_INT4) {
        {
          const f32x8 z0a = fac8(1, 8 * hl), z0b = fac8(1, 16 + 8 * hl);
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            c0[r] = fmaf(c0[r], s0a[r], fmaf(z0a[r], qsum, neg_m));
            c0[8 + r] = fmaf(c0[8 + r], s0b[r], fmaf(z0b[r], qsum, neg_m));
          }
        }
        {
          const f32x8 z1a = fac8(1, 32 + 8 * hl), z1b = fac8(1, 48 + 8 * hl);
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            c1[r] = fmaf(c1[r], s1a[r], fmaf(z1a[r], qsum, neg_m));
            c1[8 + r] = fmaf(c1[8 + r], s1b[r], fmaf(z1b[r], qsum, neg_m));
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          c0[r] = fmaf(c0[r], s0a[r], neg_m);
          c0[8 + r] = fmaf(c0[8 + r], s0b[r], neg_m);
          c1[r] = fmaf(c1[r], s1a[r], neg_m);
          c1[8 + r] = fmaf(c1[8 + r], s1b[r], neg_m);
        }
      }
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
    // Lazy rescale, only when a row's maximum passes m_run + RESCALE_SLACK
    // (or its first visible key arrives): m_run moves up by mx, and the
    // tile's relative logits move down by the same amount.
    const bool need = (m_run == -INFINITY) ? (mx != -INFINITY) : (mx > RESCALE_SLACK);
    if (__ballot(need)) {
      const float shift = need ? mx : 0.f;
      const float alpha = (need && m_run != -INFINITY) ? __builtin_amdgcn_exp2f(-mx) : 1.f;
      l_run *= alpha;
      u_run *= alpha;
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] *= alpha;
      if (need) m_run = mx - neg_m;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        c0[r] -= shift;
        c1[r] -= shift;
      }
    }
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
        const float p00 = __builtin_amdgcn_exp2f(c0[r]);
        const float p01 = __builtin_amdgcn_exp2f(c0[8 + r]);
        const float p10 = __builtin_amdgcn_exp2f(c1[r]);
        const float p11 = __builtin_amdgcn_exp2f(c1[8 + r]);
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
      compute_tile(t, kb, vb, fac, [] {});
      if (t + 1 >= ntiles) break;
      wait_dma_and_sync();  // codes(t+1) in slot 1
      if (t + 2 < ntiles) issue_codes(t + 2, kc0, vc0, fc0);
      widen_tile(t + 1, kc1, vc1, fc1, kb, vb, fac);
      lds_barrier();
      compute_tile(t + 1, kb, vb, fac, [] {});
    }
  } else {
    // ---- tile t (codes slot and bf16 buffer t & 1), one barrier each:
    //      [widen(t) done, codes(t+1) landed, compute(t-1) done] barrier,
    //      DMA codes(t+2) into the slot widen(t) read, compute(t) with
    //      widen(t+1) after its S MFMAs (buffer (t+1) & 1 was last read by
    //      compute(t-1), before the barrier)
    if (ntiles > 0) {
      issue_codes(0, kc0, vc0, fc0);
      wait_dma_and_sync();
      if (ntiles > 1) issue_codes(1, kc1, vc1, fc1);
      widen_tile(0, kc0, vc0, fc0, kbs[0], vbs[0], facs[0]);
    }
    for (int t = 0; t < ntiles; t += 2) {
      wait_dma_and_sync();
      if (t + 2 < ntiles) issue_codes(t + 2, kc0, vc0, fc0);
      compute_tile(t, kbs[0], vbs[0], facs[0], [&] {
        if (t + 1 < ntiles) widen_tile(t + 1, kc1, vc1, fc1, kbs[1], vbs[1], facs[1]);
      });
      if (t + 1 >= ntiles) break;
      wait_dma_and_sync();
      if (t + 3 < ntiles) issue_codes(t + 3, kc1, vc1, fc1);
      compute_tile(t + 1, kbs[1], vbs[1], facs[1], [&] {
        if (t + 2 < ntiles) widen_tile(t + 2, kc0, vc0, fc0, kbs[0], vbs[0], facs[0]);
      });
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

}  // namespace

hipError_t launch_attn_a_quant_d128(const AttnArgs &a, hipStream_t s) {
  const int groups = a.B * a.Hkv;
  const int R = a.qg * a.T;
  const int nA = groups * ((R + 127) / 128) * a.nsplit;
  KernelTimer timer(H2O_K_ATTN_A, s);
  if (R <= 16) return launch_attn_a_short_d128(a, s);  // short chunks: all formats, attn_short.hip
  auto launch_long = [&](auto fmt_tag) {
    constexpr int FMT = decltype(fmt_tag)::value;
    if (R >= 256) {  // long chunks: 256 rows per block share each widened tile
      const int n8 = groups * ((R + 255) / 256) * a.nsplit;
      hipLaunchKernelGGL((attn_a_quant<FMT, 8>), dim3(n8), dim3(512), 0, s, a);
    } else {
      hipLaunchKernelGGL((attn_a_quant<FMT, 4>), dim3(nA), dim3(256), 0, s, a);
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
