// Pass A for short chunks (at most 16 packed query rows per KV group, bf16
// queries, head dimension 128), for bf16, 8-bit and 4-bit caches.
//
// Same mathematics as the other attention passes ("Learning how to Forget",
// §A.7: softmax of mask(d_h^{-1/2} Q K^T), output Y = m V; §A.1 mask with the
// chunk attending before it is written).  8/4-bit caches are read as codes
// (x = c s, or c s + z per slot): the products run on the codes and the
// per-slot factors are applied outside them,
//   logit_ij = s_j <q_i, c_j> (+ z_j sum(q_i)),
//   out_i    = sum_j (P_ij s_j) c_j (+ sum_j P_ij z_j, the same for every d).
//
// Each wavefront takes 16 keys of every 64-key tile of its key split on 16x16
// MFMAs (S^T = K Q^T with keys as rows, O^T += V^T P^T), keeps its own running
// max and sum, and the four wavefronts merge through LDS at the end (the
// rescaling the key-split combine applies).  The rows go HBM -> registers with
// plain loads, NPF tiles ahead, and codes widen in registers straight into the
// MFMA operands: nothing passes through LDS between load and use, and no
// wavefront waits for another inside the tile loop.  The pace is set by the
// per-tile instruction chain (widening, products, softmax), not by the loads:
// with the loads taken out the 8/4-bit pass is about as slow, and rings deeper
// than two tiles or eight wavefronts per block measured slower.
//
// Head-dimension order inside the products.  One permutation of d applied
// to both operands of S = K Q^T leaves every dot product unchanged, and one
// applied to V's columns only relabels O's; both are chosen so that a lane's
// share of an operand is contiguous in a cache row:
//   S (steps st = 0..3 of 16x16x32): lane (n, g) = (lane % 16, lane / 16)
//     supplies key n and query row n at d = 32 g + 8 st + e, e = 0..7;
//   O^T += V^T P^T (blocks k = 0..7 of 16x16x16): lane (m, g) supplies
//     d = 8 m + k of keys 4 g + i, i = 0..3 (bytes 16m.. of a bf16 row, 8m..
//     of an 8-bit code row, 4m.. of a 4-bit one); its accumulator register i
//     of block k then holds d = 32 g + 8 i + k of query row lane % 16.

#include <type_traits>

#include "code_widen.hpp"
#include "device_util.hpp"
#include "h2o_internal.hpp"
#include "tile_util.hpp"

namespace h2o {
namespace {

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

// Bytes of one cache row: bf16 values or codes.
template <int FMT>
constexpr int row_bytes() {
  return FMT == FMT_NATIVE ? 2 * D : QTile<FMT>::CODE_ROW;
}

// One lane's share of one tile wholly in the cache, as loaded.
template <int FMT>
struct DecShare {
  static constexpr int KW = row_bytes<FMT>() / 64;    // 16-byte words of key n (d = 32g ..)
  static constexpr int VW = row_bytes<FMT>() / 16;    // 32-bit words of keys 4g + i (d = 8m ..)
  static constexpr int NF = FMT == FMT_NATIVE ? 0 : FMT == FMT_INT8 ? 2 : 4;  // ks, vs (, kz, vz)
  uint4 k[KW];
  uint32_t v[VW];
  uint2 f[NF > 0 ? NF : 1];  // fp16 factors of keys 4g .. 4g + 3
};

template <int FMT, bool LG, int NPF, int NW>
__global__ __launch_bounds__(64 * NW, NW / 2) void attn_a_short(AttnArgs a) {
  using Sh = DecShare<FMT>;
  constexpr int CODE_ROW = row_bytes<FMT>();
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
      if constexpr (FMT == FMT_NATIVE) {
        const uint4 x = *reinterpret_cast<const uint4 *>(vp);
        s.v[4 * i] = x.x;
        s.v[4 * i + 1] = x.y;
        s.v[4 * i + 2] = x.z;
        s.v[4 * i + 3] = x.w;
      } else if constexpr (FMT == FMT_INT8) {
        const uint2 x = *reinterpret_cast<const uint2 *>(vp);
        s.v[2 * i] = x.x;
        s.v[2 * i + 1] = x.y;
      } else {
        s.v[i] = *reinterpret_cast<const uint32_t *>(vp);
      }
    }
    // four consecutive fp16 factors, 8-byte aligned only when C % 4 == 0; the
    // copy states 2-byte alignment and the compiler still issues one 8-byte load
    // (the parity tests include capacities that are not a multiple of 4)
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
    // c[i]: tile key kk0 + i of row n; factors bring it to log2 units.  The
    // stored logits are q.k for bf16 caches (the weight pass scales them) and
    // already in log2 units for 8/4-bit ones.
    auto store_logits4 = [&] {
      if constexpr (LG) {
        H2O_DEVICE_CHECK(grp < a.B * a.Hkv && j0 + kk0 + 3 < a.lg_stride);
        if (row_ok)
          *reinterpret_cast<float4 *>(a.lg + (static_cast<size_t>(grp) * R + n) * a.lg_stride + j0 + kk0) =
              make_float4(c[0], c[1], c[2], c[3]);
      }
    };
    if constexpr (FMT == FMT_NATIVE) store_logits4();
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = (FMT == FMT_INT4) ? fmaf(c[i], sk[i], zk[i] * qsum) : c[i] * sk[i];
    if constexpr (FMT != FMT_NATIVE) store_logits4();
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
    if constexpr (FMT != FMT_NATIVE) {
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] *= sv[i];
    }
    const i16x4 pb = __builtin_bit_cast(i16x4, make_uint2(pack_bf16_hw(p[0], p[1]), pack_bf16_hw(p[2], p[3])));
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop(k), pb, o[k], 0, 0, 0);
  };

  // a tile wholly in the cache, from its loaded share
  auto full_tile = [&](int tile, const Sh &s) {
    if constexpr (FMT == FMT_NATIVE) {
      const float sk[4] = {a.sl2, a.sl2, a.sl2, a.sl2}, zero[4] = {0.f, 0.f, 0.f, 0.f};
      const uint4 kw[4] = {s.k[0], s.k[1], s.k[2], s.k[3]};
      tile_body(tile, kw, sk, zero, zero, zero, [&](int k) {
        // element k of the four rows' words (row i: s.v[4i .. 4i+3])
        const uint32_t sel = (k & 1) ? 0x07060302u : 0x05040100u;
        const int w = k >> 1;
        return __builtin_bit_cast(i16x4, make_uint2(__builtin_amdgcn_perm(s.v[4 + w], s.v[w], sel),
                                                    __builtin_amdgcn_perm(s.v[12 + w], s.v[8 + w], sel)));
      }, std::false_type{});
      return;
    } else {
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
    }
  };

  // any other tile: codes of rows below n_occ, new keys (bf16) above, zeros
  // past the chunk
  auto tail_tile = [&](int tile) {
    const int j0 = (t_lo + tile) * 64;
    const int jk = j0 + 16 * wq + n;  // key row of the lane's K operand
    uint4 kw[4];
    if (jk < n_occ) {
      const char *kp = kcb + (cache_row0 + jk) * CODE_ROW + g4 * (CODE_ROW / 4);
      if constexpr (FMT == FMT_NATIVE) {
#pragma unroll
        for (int st = 0; st < 4; ++st) kw[st] = *reinterpret_cast<const uint4 *>(kp + 16 * st);
      } else {
        widen32<FMT, FMT == FMT_INT4>(kp, kw);
      }
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
        const char *vp = vcb + row * CODE_ROW + n * (CODE_ROW / 16);
        zk[i] = zv[i] = 0.f;
        if constexpr (FMT == FMT_NATIVE) {
          vrow[i] = *reinterpret_cast<const uint4 *>(vp);
          sk[i] = a.sl2;
          sv[i] = 1.f;
          continue;
        }
        vrow[i] = widen8<FMT>(vp);
        const float s_k = f16_to_f32(a.ks[row]);
        sk[i] = s_k * a.sl2;
        sv[i] = f16_to_f32(a.vs[row]);
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
  H2O_DEVICE_CHECK(lr < plane && split < a.nsplit);
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

hipError_t launch_attn_a_short_d128(const AttnArgs &a, hipStream_t s) {
  // tiles each wavefront keeps in flight (8 / 4 / 2 KB of rows each for
  // bf16 / 8-bit / 4-bit caches) and wavefronts per block
  constexpr int NPF = 2, NW = 4;
  const dim3 grid(a.B * a.Hkv * a.nsplit), block(64 * NW);
  auto go = [&](auto fmt_tag) {
    constexpr int FMT = decltype(fmt_tag)::value;
    if (a.lg) {
      hipLaunchKernelGGL((attn_a_short<FMT, true, NPF, NW>), grid, block, 0, s, a);
    } else {
      hipLaunchKernelGGL((attn_a_short<FMT, false, NPF, NW>), grid, block, 0, s, a);
    }
  };
  if (a.cache_fmt == FMT_INT8) {
    go(std::integral_constant<int, FMT_INT8>{});
  } else if (a.cache_fmt == FMT_INT4) {
    go(std::integral_constant<int, FMT_INT4>{});
  } else {
    go(std::integral_constant<int, FMT_NATIVE>{});
  }
  return hipGetLastError();
}

}  // namespace h2o
