// bf16 matrix-core attention passes for gfx950 (v_mfma_f32_32x32x16_bf16).
//
// Pass A (one block = 128 packed query rows of one KV group, 4 wavefronts x 32
// rows): flash-style forward.  S^T = K Q^T per 64-key tile from LDS, online
// softmax in the log2 domain with lazy rescaling, O^T += V^T P^T with P in
// bf16.  Writes out and the row normaliser L = m + log2(l).
//   ("Learning how to Forget", §A.7: Y = softmax(mask(d_h^{-1/2} Q K^T)) V.)
// Pass B (one block = 128 keys of one KV group, 4 wavefronts x 32 keys):
// recomputes S = Q K^T for every query row of the group, streaming 64-row Q
// blocks through LDS, and sums exp2(x - L) per key in fp32 with compensated
// accumulation -> exact summed weights, never materialising the T x S matrix.
//   (§3.1.1 / §A.7: summed attention weights, here reduced over the q_g heads
//   of the group as the H2O score is kept per KV head.)
//
// Query rows of a group are packed as r = i*q_g + hh (chunk position i, head
// hh of the group), so one K/V tile in LDS serves all heads of the group.
// Keys of a group are the n_occ cache slots followed by the T chunk keys; a
// chunk key t is visible to row r iff t <= i (cache slots are all visible).
//
// Quantised caches (int8: x = c*s; int4: x = c*s + z, per slot): codes are
// exact in bf16, so tiles are staged as bf16 codes and the per-slot scale is
// applied outside the matrix product: logits = s_j <q, c_j> (+ z_j sum(q)),
// and P'_ij = P_ij * s_j before the PV product (+ sum_j P_ij z_j per row).
// The chunk's own keys/values are used at input precision.
//
// MFMA operand layouts (32x32x16, wave64): A[m][k] lane = m + 32*(k/8),
// element k%8; B[k][n] lane = n + 32*(k/8), element k%8; C[m][n] lane = n +
// 32*((m/4)%2), register 4*(m/8) + m%4.

#include "device_util.hpp"
#include "h2o_internal.hpp"

namespace h2o {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int A_ROWS = 128;  // packed query rows per pass-A block
constexpr int A_KT = 64;     // keys per pass-A tile
constexpr int VSTR = A_KT + 8;  // row stride (elements) of the transposed V tile
constexpr int B_KEYS = 128;  // keys per pass-B block
constexpr int B_RB = 64;     // query rows per pass-B LDS block
constexpr float RESCALE_SLACK = 8.f;  // allowed growth of exp2 arguments before rescaling

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds16(const char *p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(p));
}

// Row-major tile of rows x D bf16 in LDS, 16-byte chunks XOR-swizzled so that
// 16 consecutive rows read at one chunk index hit 16 distinct bank groups.
template <int D>
__device__ __forceinline__ int tile_off(int row, int chunk) {
  if constexpr (D == 128) {
    return row * 256 + ((chunk ^ (row & 15)) << 4);
  } else {
    return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4);
  }
}

// A-operand row m of S^T = K Q^T holds key perm(m) (bits 2 and 3 swapped), so
// that accumulator registers 0..7 / 8..15 of lane half h hold keys 8h..8h+7 /
// 16+8h..16+8h+7 -- exactly the k-order the P^T operand of the PV product needs.
__device__ __forceinline__ int perm_key(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

__device__ __forceinline__ uint32_t pack_bf16_hi(float lo, float hi) {
  // bf16 truncation of two fp32 values known to be exact in bf16 (small integers)
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

__device__ __forceinline__ uint32_t pack_bf16_rne(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// 16 int8 codes -> 16 bf16 (exact), as two 16-byte chunks.
__device__ __forceinline__ void i8x16_to_bf16(uint4 c, uint4 &o0, uint4 &o1) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  uint32_t r[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int32_t x = static_cast<int32_t>(w[q]);
    const float f0 = static_cast<float>((x << 24) >> 24);
    const float f1 = static_cast<float>((x << 16) >> 24);
    const float f2 = static_cast<float>((x << 8) >> 24);
    const float f3 = static_cast<float>(x >> 24);
    r[2 * q] = pack_bf16_hi(f0, f1);
    r[2 * q + 1] = pack_bf16_hi(f2, f3);
  }
  o0 = make_uint4(r[0], r[1], r[2], r[3]);
  o1 = make_uint4(r[4], r[5], r[6], r[7]);
}

// 8 int4 codes (one dword, element 2k in the low nibble of byte k) -> 8 bf16.
__device__ __forceinline__ uint4 u4x8_to_bf16(uint32_t c) {
  uint32_t r[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t byte = (c >> (8 * q)) & 0xffu;
    r[q] = pack_bf16_hi(static_cast<float>(byte & 15u), static_cast<float>(byte >> 4));
  }
  return make_uint4(r[0], r[1], r[2], r[3]);
}

// ---------------------------------------------------------------------------
// Pass A
// ---------------------------------------------------------------------------

template <int FMT, int D>
struct PassA {
  static constexpr int NST = D / 16;                 // 16-wide k steps over D
  static constexpr int NBLK = D / 32;                // 32-wide output blocks over D
  static constexpr int KS_BYTES = A_KT * D * 2;      // K tile, bf16
  static constexpr int VT_BYTES = D * VSTR * 2;      // V^T tile, bf16
  static constexpr int SC_BYTES = (FMT == FMT_NATIVE) ? 0 : 4 * A_KT * 4;
  static constexpr int BUF = KS_BYTES + VT_BYTES + SC_BYTES;
  static constexpr int LDS = 2 * BUF;
  static constexpr int KCH = A_KT * D / 8 / 256;     // K 16-byte bf16 chunks per thread
  static constexpr int V_THREADS = 2 * D;            // threads staging V (4 keys x 8 d each)
};

template <int FMT, int D>
__global__ __launch_bounds__(256, 2) void attn_a_mfma(AttnArgs a) {
  using P = PassA<FMT, D>;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, hl = lane >> 5;
  const int R = a.qg * a.T;
  const int tiles_per_grp = (R + A_ROWS - 1) / A_ROWS;
  const int wi_all = xcd_remap(blockIdx.x, gridDim.x);
  const int split = wi_all % a.nsplit;  // key split of this block (0 when unsplit)
  const int wi = wi_all / a.nsplit;
  // Row blocks go out last first: under the causal mask the last rows see the
  // most keys, and starting the longest blocks first evens out the tail.
  const int grp = wi / tiles_per_grp, rt = tiles_per_grp - 1 - wi % tiles_per_grp;
  const int g = grp % a.Hkv, b = grp / a.Hkv;
  const int row0 = rt * A_ROWS;
  const int my_row = row0 + wave * 32 + n;
  const bool row_ok = my_row < R;
  const int i_q = row_ok ? my_row / a.qg : 0;
  const int h_q = g * a.qg + (row_ok ? my_row % a.qg : 0);
  const int n_occ = a.n_occ;

  // Q^T fragments (B operand): lane (n, hl) holds Q[row n][16 st + 8 hl + 0..7]
  bf16x8 qf[P::NST];
  float qsum = 0.f;
  {
    const uint16_t *qrow =
        static_cast<const uint16_t *>(a.q) + ((static_cast<size_t>(b) * a.Hq + h_q) * a.T + i_q) * D;
#pragma unroll
    for (int st = 0; st < P::NST; ++st) {
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

  const int last_row = min(R, row0 + A_ROWS) - 1;
  const int key_end = n_occ + last_row / a.qg + 1;  // keys any row of the block can see
  // key tiles t_lo .. t_lo + ntiles - 1 (all of them when unsplit)
  const int ntiles_all = (key_end + A_KT - 1) / A_KT;
  int t_lo, ntiles;  // key tiles t_lo .. t_lo + ntiles - 1 of this split (ntiles 0: none)
  split_tiles(ntiles_all, a.nsplit, split, t_lo, ntiles);
  const size_t cache_row0 = static_cast<size_t>(grp) * a.C;
  const size_t new_row0 = static_cast<size_t>(grp) * a.T;

  // ---- staging registers ----
  uint4 kst[P::KCH];
  uint4 vst[4];
  float sc_st[4];
  const int vkg = tid & 15, vch = tid >> 4;  // V staging: keys 4*vkg.., d chunk vch

  auto load_tile = [&](int j0) {
    if constexpr (FMT == FMT_NATIVE) {
#pragma unroll
      for (int q = 0; q < P::KCH; ++q) {
        const int e = tid + 256 * q;
        const int row = e / (D / 8), c = e % (D / 8);
        const int j = j0 + row;
        const uint16_t *src = nullptr;
        if (j < n_occ) {
          src = static_cast<const uint16_t *>(a.kc) + (cache_row0 + j) * D;
        } else if (j - n_occ < a.T) {
          src = static_cast<const uint16_t *>(a.kn) + (new_row0 + (j - n_occ)) * D;
        }
        kst[q] = src ? *reinterpret_cast<const uint4 *>(src + 8 * c) : make_uint4(0, 0, 0, 0);
      }
    } else {
      // one thread per (key, 8-element chunk of d); cache keys fetch codes
#pragma unroll
      for (int q = 0; q < P::KCH; ++q) {
        const int e = tid + 256 * q;
        const int row = e / (D / 8), c = e % (D / 8);
        const int j = j0 + row;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (j < n_occ) {
          if constexpr (FMT == FMT_INT8) {
            const uint2 codes = *reinterpret_cast<const uint2 *>(
                static_cast<const int8_t *>(a.kc) + (cache_row0 + j) * D + 8 * c);
            uint4 lo, hi;
            i8x16_to_bf16(make_uint4(codes.x, codes.y, 0, 0), lo, hi);
            v = lo;
          } else {
            const uint32_t codes = *reinterpret_cast<const uint32_t *>(
                static_cast<const uint8_t *>(a.kc) + (cache_row0 + j) * (D / 2) + 4 * c);
            v = u4x8_to_bf16(codes);
          }
        } else if (j - n_occ < a.T) {
          v = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.kn) +
                                               (new_row0 + (j - n_occ)) * D + 8 * c);
        }
        kst[q] = v;
      }
    }
    if (tid < P::V_THREADS) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = j0 + 4 * vkg + r;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (j < n_occ) {
          if constexpr (FMT == FMT_NATIVE) {
            v = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.vc) +
                                                 (cache_row0 + j) * D + 8 * vch);
          } else if constexpr (FMT == FMT_INT8) {
            const uint2 codes = *reinterpret_cast<const uint2 *>(
                static_cast<const int8_t *>(a.vc) + (cache_row0 + j) * D + 8 * vch);
            uint4 lo, hi;
            i8x16_to_bf16(make_uint4(codes.x, codes.y, 0, 0), lo, hi);
            v = lo;
          } else {
            const uint32_t codes = *reinterpret_cast<const uint32_t *>(
                static_cast<const uint8_t *>(a.vc) + (cache_row0 + j) * (D / 2) + 4 * vch);
            v = u4x8_to_bf16(codes);
          }
        } else if (j - n_occ < a.T) {
          v = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.vn) +
                                               (new_row0 + (j - n_occ)) * D + 8 * vch);
        }
        vst[r] = v;
      }
    }
    if constexpr (FMT != FMT_NATIVE) {
      // per-key factors: [0] sl2*s_k, [1] sl2*z_k, [2] s_v, [3] z_v (chunk keys: 1, 0)
      if (tid < A_KT) {
        const int j = j0 + tid;
        float ks = 1.f, kz = 0.f, vs = 1.f, vz = 0.f;
        if (j < n_occ) {
          ks = f16_to_f32(a.ks[cache_row0 + j]);
          vs = f16_to_f32(a.vs[cache_row0 + j]);
          if constexpr (FMT == FMT_INT4) {
            kz = f16_to_f32(a.kz[cache_row0 + j]);
            vz = f16_to_f32(a.vz[cache_row0 + j]);
          }
        }
        sc_st[0] = ks * a.sl2;
        sc_st[1] = kz * a.sl2;
        sc_st[2] = vs;
        sc_st[3] = vz;
      }
    }
  };

  auto store_tile = [&](int buf) {
    char *kb = smem + buf * P::BUF;
    char *vb = kb + P::KS_BYTES;
#pragma unroll
    for (int q = 0; q < P::KCH; ++q) {
      const int e = tid + 256 * q;
      const int row = e / (D / 8), c = e % (D / 8);
      *reinterpret_cast<uint4 *>(kb + tile_off<D>(row, c)) = kst[q];
    }
    if (tid < P::V_THREADS) {
      // transpose 4 keys x 8 d -> 8 rows (d) of 4 keys
      const uint32_t w[4][4] = {{vst[0].x, vst[0].y, vst[0].z, vst[0].w},
                                {vst[1].x, vst[1].y, vst[1].z, vst[1].w},
                                {vst[2].x, vst[2].y, vst[2].z, vst[2].w},
                                {vst[3].x, vst[3].y, vst[3].z, vst[3].w}};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int odd = 0; odd < 2; ++odd) {
          const uint32_t sel = odd ? 0x07060302u : 0x05040100u;
          const uint32_t lo = __builtin_amdgcn_perm(w[1][q], w[0][q], sel);
          const uint32_t hi = __builtin_amdgcn_perm(w[3][q], w[2][q], sel);
          const int d = 8 * vch + 2 * q + odd;
          *reinterpret_cast<uint2 *>(vb + (d * VSTR + 4 * vkg) * 2) = make_uint2(lo, hi);
        }
      }
    }
    if constexpr (FMT != FMT_NATIVE) {
      float *sb = reinterpret_cast<float *>(vb + P::VT_BYTES);
      if (tid < A_KT) {
        sb[tid] = sc_st[0];
        sb[A_KT + tid] = sc_st[1];
        sb[2 * A_KT + tid] = sc_st[2];
        sb[3 * A_KT + tid] = sc_st[3];
      }
    }
  };

  f32x16 o[P::NBLK];
#pragma unroll
  for (int k = 0; k < P::NBLK; ++k) o[k] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f, u_run = 0.f;
  const int prow = perm_key(n);

  if (ntiles > 0) {
    load_tile(t_lo * A_KT);
    store_tile(0);
    __syncthreads();
  }

  for (int t = 0; t < ntiles; ++t) {
    const int j0 = (t_lo + t) * A_KT;
    if (t + 1 < ntiles) load_tile(j0 + A_KT);
    const char *kb = smem + (t & 1) * P::BUF;
    const char *vb = kb + P::KS_BYTES;

    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int st = 0; st < P::NST; ++st) {
      const bf16x8 k0 = lds16(kb + tile_off<D>(prow, 2 * st + hl));
      const bf16x8 k1 = lds16(kb + tile_off<D>(32 + prow, 2 * st + hl));
      s0 = mfma32(k0, qf[st], s0);
      s1 = mfma32(k1, qf[st], s1);
    }

    // logits in log2 units: x = s * factor_j (+ z-term)
    float x0[16], x1[16];
    if constexpr (FMT == FMT_NATIVE) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        x0[r] = s0[r];
        x1[r] = s1[r];
      }
    } else {
      const float *sb = reinterpret_cast<const float *>(vb + P::VT_BYTES);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kt = 16 * (r >> 3) + 8 * hl + (r & 7);
        if constexpr (FMT == FMT_INT8) {
          x0[r] = s0[r] * sb[kt];
          x1[r] = s1[r] * sb[32 + kt];
        } else {
          x0[r] = fmaf(s0[r], sb[kt], sb[A_KT + kt] * qsum);
          x1[r] = fmaf(s1[r], sb[32 + kt], sb[A_KT + 32 + kt] * qsum);
        }
      }
    }
    if (j0 + A_KT > n_occ || !row_ok) {  // tile reaches the chunk keys: causal mask
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kt = 16 * (r >> 3) + 8 * hl + (r & 7);
        const int ja = j0 + kt, jb = ja + 32;
        if (!row_ok || (ja >= n_occ && ja - n_occ > i_q)) x0[r] = -INFINITY;
        if (!row_ok || (jb >= n_occ && jb - n_occ > i_q)) x1[r] = -INFINITY;
      }
    }
    float mx = x0[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, x0[r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, x1[r]);
    if constexpr (FMT == FMT_NATIVE) mx *= a.sl2;
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (__ballot(mx > m_run + RESCALE_SLACK)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      if constexpr (FMT == FMT_INT4) u_run *= alpha;
#pragma unroll
      for (int k = 0; k < P::NBLK; ++k) o[k] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;

    float p0[16], p1[16];
    float ls = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if constexpr (FMT == FMT_NATIVE) {
        p0[r] = __builtin_amdgcn_exp2f(fmaf(x0[r], a.sl2, -m_use));
        p1[r] = __builtin_amdgcn_exp2f(fmaf(x1[r], a.sl2, -m_use));
      } else {
        p0[r] = __builtin_amdgcn_exp2f(x0[r] - m_use);
        p1[r] = __builtin_amdgcn_exp2f(x1[r] - m_use);
      }
      ls += p0[r] + p1[r];
    }
    l_run += ls;
    if constexpr (FMT != FMT_NATIVE) {
      const float *sb = reinterpret_cast<const float *>(vb + P::VT_BYTES);
      float us = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kt = 16 * (r >> 3) + 8 * hl + (r & 7);
        if constexpr (FMT == FMT_INT4) {
          us = fmaf(p0[r], sb[3 * A_KT + kt], us);
          us = fmaf(p1[r], sb[3 * A_KT + 32 + kt], us);
        }
        p0[r] *= sb[2 * A_KT + kt];
        p1[r] *= sb[2 * A_KT + 32 + kt];
      }
      if constexpr (FMT == FMT_INT4) u_run += us;
    }
    bf16x8 pb[4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pb[0][e] = static_cast<__bf16>(p0[e]);
      pb[1][e] = static_cast<__bf16>(p0[8 + e]);
      pb[2][e] = static_cast<__bf16>(p1[e]);
      pb[3][e] = static_cast<__bf16>(p1[8 + e]);
    }
#pragma unroll
    for (int blk = 0; blk < P::NBLK; ++blk) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 va = lds16(vb + ((32 * blk + n) * VSTR + 16 * ks + 8 * hl) * 2);
        o[blk] = mfma32(va, pb[ks], o[blk]);
      }
    }
    if (t + 1 < ntiles) store_tile((t + 1) & 1);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  float u_tot = 0.f;
  if constexpr (FMT == FMT_INT4) u_tot = u_run + __shfl_xor(u_run, 32);
  if (!row_ok) return;
  const size_t li = (static_cast<size_t>(b) * a.Hq + h_q) * a.T + i_q;
  if (a.nsplit > 1) {  // unnormalised partial output and (m, l) of this key split
    const size_t pr = static_cast<size_t>(split) * a.B * a.Hq * a.T + li;
    float *po = a.part + pr * D;
#pragma unroll
    for (int blk = 0; blk < P::NBLK; ++blk) {
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
  for (int blk = 0; blk < P::NBLK; ++blk) {
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int d = 32 * blk + 8 * a4 + 4 * hl;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (o[blk][4 * a4 + e] + u_tot) * inv;
      *reinterpret_cast<uint2 *>(orow + d) = make_uint2(pack_bf16_rne(v[0], v[1]), pack_bf16_rne(v[2], v[3]));
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
// Pass B
// ---------------------------------------------------------------------------

template <int D>
struct PassB {
  static constexpr int NST = D / 16;
  static constexpr int QB_BYTES = B_RB * D * 2;
  static constexpr int BUF = QB_BYTES + 2 * B_RB * 4;  // Q rows + L + sum(q)
  static constexpr int LDS = 2 * BUF;
  static constexpr int QCH = B_RB * D / 8 / 256;  // 16-byte chunks per thread
};

template <int FMT, int D>
__global__ __launch_bounds__(256, 2) void attn_b_mfma(AttnArgs a) {
  using P = PassB<D>;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, hl = lane >> 5;
  const int n_occ = a.n_occ;
  const int n_keys = n_occ + a.T;
  const int R = a.qg * a.T;
  const int kblocks = (n_keys + B_KEYS - 1) / B_KEYS;
  const int wi = xcd_remap(blockIdx.x, gridDim.x);
  const int grp = wi / kblocks, kbk = wi % kblocks;
  const int g = grp % a.Hkv, b = grp / a.Hkv;
  const int j_base = kbk * B_KEYS;
  const int my_key = j_base + wave * 32 + n;
  const bool key_ok = my_key < n_keys;
  const int tnew = my_key - n_occ;  // >= 0 for a chunk key
  const size_t cache_row = static_cast<size_t>(grp) * a.C + my_key;
  const size_t lse_plane = static_cast<size_t>(a.B) * a.Hq * a.T;

  // K^T fragments (B operand): lane (n, hl) holds K[key n][16 st + 8 hl + 0..7]
  bf16x8 kf[P::NST];
  float fk = a.sl2, fz = 0.f;
#pragma unroll
  for (int st = 0; st < P::NST; ++st) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (key_ok) {
      if (tnew < 0) {
        if constexpr (FMT == FMT_NATIVE) {
          v = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.kc) + cache_row * D +
                                               16 * st + 8 * hl);
        } else if constexpr (FMT == FMT_INT8) {
          const uint2 codes = *reinterpret_cast<const uint2 *>(static_cast<const int8_t *>(a.kc) +
                                                               cache_row * D + 16 * st + 8 * hl);
          uint4 lo, hi;
          i8x16_to_bf16(make_uint4(codes.x, codes.y, 0, 0), lo, hi);
          v = lo;
        } else {
          const uint32_t codes = *reinterpret_cast<const uint32_t *>(
              static_cast<const uint8_t *>(a.kc) + cache_row * (D / 2) + 8 * st + 4 * hl);
          v = u4x8_to_bf16(codes);
        }
      } else {
        v = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.kn) +
                                             (static_cast<size_t>(grp) * a.T + tnew) * D + 16 * st + 8 * hl);
      }
    }
    kf[st] = __builtin_bit_cast(bf16x8, v);
  }
  if constexpr (FMT != FMT_NATIVE) {
    if (key_ok && tnew < 0) {
      fk = f16_to_f32(a.ks[cache_row]) * a.sl2;
      if constexpr (FMT == FMT_INT4) fz = f16_to_f32(a.kz[cache_row]) * a.sl2;
    }
  }

  // rows before the block's first chunk key cannot see any key of it
  const int row_first = (j_base >= n_occ) ? (j_base - n_occ) * a.qg : 0;
  const int rb_begin = row_first / B_RB * B_RB;
  const int nrb = (R - rb_begin + B_RB - 1) / B_RB;
  const int t_last = j_base + B_KEYS - 1 - n_occ;  // largest chunk index of the block's keys

  uint4 qst[P::QCH];
  float lst = 0.f, sst = 0.f;
  auto load_rows = [&](int rb) {
#pragma unroll
    for (int q = 0; q < P::QCH; ++q) {
      const int e = tid + 256 * q;
      const int rr = e / (D / 8), c = e % (D / 8);
      const int row = rb + rr;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row < R) {
        const int ii = row / a.qg, hh = g * a.qg + row % a.qg;
        v = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.q) +
                                             ((static_cast<size_t>(b) * a.Hq + hh) * a.T + ii) * D + 8 * c);
      }
      qst[q] = v;
    }
    if (tid < B_RB) {
      const int row = rb + tid;
      lst = 0.f;
      sst = 0.f;
      if (row < R) {
        const int ii = row / a.qg, hh = g * a.qg + row % a.qg;
        const size_t li = (static_cast<size_t>(b) * a.Hq + hh) * a.T + ii;
        lst = a.lse2[li];
        if constexpr (FMT == FMT_INT4) sst = a.lse2[lse_plane + li];
      }
    }
  };
  auto store_rows = [&](int buf) {
    char *qb = smem + buf * P::BUF;
#pragma unroll
    for (int q = 0; q < P::QCH; ++q) {
      const int e = tid + 256 * q;
      const int rr = e / (D / 8), c = e % (D / 8);
      *reinterpret_cast<uint4 *>(qb + tile_off<D>(rr, c)) = qst[q];
    }
    if (tid < B_RB) {
      float *lb = reinterpret_cast<float *>(qb + P::QB_BYTES);
      lb[tid] = lst;
      lb[B_RB + tid] = sst;
    }
  };

  float acc = 0.f, comp = 0.f;
  load_rows(rb_begin);
  store_rows(0);
  __syncthreads();
  for (int it = 0; it < nrb; ++it) {
    const int rb = rb_begin + it * B_RB;
    if (it + 1 < nrb) load_rows(rb + B_RB);
    const char *qb = smem + (it & 1) * P::BUF;
    const float *lb = reinterpret_cast<const float *>(qb + P::QB_BYTES);
    const bool full = (rb + B_RB <= R) && (j_base + B_KEYS <= n_occ || rb / a.qg >= t_last);
    float part = 0.f;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      f32x16 s = f32x16{};
#pragma unroll
      for (int st = 0; st < P::NST; ++st) {
        const bf16x8 qa = lds16(qb + tile_off<D>(32 * sub + n, 2 * st + hl));
        s = mfma32(qa, kf[st], s);
      }
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int rr0 = 32 * sub + 8 * a4 + 4 * hl;
        const float4 L = *reinterpret_cast<const float4 *>(lb + rr0);
        float4 Sq = make_float4(0.f, 0.f, 0.f, 0.f);
        if constexpr (FMT == FMT_INT4) Sq = *reinterpret_cast<const float4 *>(lb + B_RB + rr0);
        const float Lv[4] = {L.x, L.y, L.z, L.w};
        const float Sv[4] = {Sq.x, Sq.y, Sq.z, Sq.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x;
          if constexpr (FMT == FMT_INT4) {
            x = fmaf(s[4 * a4 + e], fk, fmaf(fz, Sv[e], -Lv[e]));
          } else {
            x = fmaf(s[4 * a4 + e], fk, -Lv[e]);
          }
          if (!full) {
            const int row = rb + rr0 + e;
            const bool vis = row < R && (tnew < 0 || tnew <= row / a.qg);
            if (!vis) x = -INFINITY;
          }
          part += __builtin_amdgcn_exp2f(x);
        }
      }
    }
    const float y = part - comp;
    const float tt = acc + y;
    comp = (tt - acc) - y;
    acc = tt;
    if (it + 1 < nrb) store_rows((it + 1) & 1);
    __syncthreads();
  }
  const float mine = acc - comp;
  const float other = __shfl_xor(mine, 32);
  if (key_ok && hl == 0) a.wsum[static_cast<size_t>(grp) * n_keys + my_key] = mine + other;
}

template <int FMT, int D>
hipError_t launch_t(const AttnArgs &a, hipStream_t s) {
  constexpr int lds_a = PassA<FMT, D>::LDS;
  constexpr int lds_b = PassB<D>::LDS;
  const int groups = a.B * a.Hkv;
  const int R = a.qg * a.T;
  const int nA = groups * ((R + A_ROWS - 1) / A_ROWS) * a.nsplit;
  static const hipError_t attr = [] {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&attn_a_mfma<FMT, D>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds_a);
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&attn_b_mfma<FMT, D>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, lds_b);
  }();
  if (attr != hipSuccess) return attr;
  auto ka = attn_a_mfma<FMT, D>;
  auto kb = attn_b_mfma<FMT, D>;
  hipError_t e;
  if (FMT != FMT_NATIVE && D == 128) {
    e = launch_attn_a_quant_d128(a, s);  // DMA-staged codes, widened in LDS
  } else {
    {
      KernelTimer timer(H2O_K_ATTN_A, s);
      hipLaunchKernelGGL(ka, dim3(nA), dim3(256), lds_a, s, a);
    }
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  if (a.nsplit > 1 && !a.lg) {  // with stored logits the weight-sum kernel merges the splits
    e = launch_attn_combine(a, s);
    if (e != hipSuccess) return e;
  }
  if (!a.wsum || (a.lg && a.defer_b)) return hipSuccess;
  if (D == 128) return a.lg ? launch_attn_b_logits(a, s) : launch_attn_b_native(a, s);  // every cache format
  const int nB = groups * ((a.n_occ + a.T + B_KEYS - 1) / B_KEYS);
  {
    KernelTimer timer(H2O_K_ATTN_B, s);
    hipLaunchKernelGGL(kb, dim3(nB), dim3(256), lds_b, s, a);
  }
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_f(const AttnArgs &a, hipStream_t s) {
  if (a.D == 64) return launch_t<FMT, 64>(a, s);
  return launch_t<FMT, 128>(a, s);
}

}  // namespace

hipError_t launch_attn_mfma(const AttnArgs &a, hipStream_t s) {
  if (a.cache_fmt == FMT_NATIVE && a.D == 128) return launch_attn_native_d128(a, s);
  switch (a.cache_fmt) {
    case FMT_INT8: return launch_f<FMT_INT8>(a, s);
    case FMT_INT4: return launch_f<FMT_INT4>(a, s);
    default: return launch_f<FMT_NATIVE>(a, s);
  }
}

}  // namespace h2o
