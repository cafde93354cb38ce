// Merge of pass A's key-split partials for short chunks (at most
// LOGIT_ROWS_MAX query rows per KV group, D = 128), done by the kernels that
// sum the stored logits (attn_b_logits, evict_cand_lg) instead of a launch of
// its own.  Split s of row r left its unnormalised output O_s and (m_s, l_s)
// (log2-domain running max and sum of its keys); the row's normaliser is
// L = M + log2(sum_s l_s 2^(m_s - M)) with M = max_s m_s, and its output
// O = sum_s 2^(m_s - M) O_s / sum_s l_s 2^(m_s - M) ("Learning how to Forget",
// §A.7: softmax over all the row's keys, here assembled from key ranges).
// Every split loop runs in a fixed order, so the result does not depend on
// which kernel merges.
#pragma once

#include "device_util.hpp"
#include "h2o_internal.hpp"

namespace h2o {

constexpr int MERGE_D = 128;  // head dimension of the short-chunk paths

// Normalisers, 16 lanes per row: lane sl of row li loads the (m, l) pairs of
// splits sl, sl + 16, sl + 32, sl + 48 (nsplit <= 64); ok false: none.
__device__ __forceinline__ void load_split_ml(const AttnArgs &a, size_t rows, size_t li, int sl, bool ok,
                                              float2 (&ml)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int sp = sl + 16 * k;
    ml[k] = (ok && sp < a.nsplit) ? *reinterpret_cast<const float2 *>(a.part_ml + 2 * (sp * rows + li))
                                  : make_float2(-INFINITY, 0.f);
  }
}

// The row's M and sum_s l_s 2^(m_s - M) across its 16 lanes (all get them);
// the lanes must be an aligned group of 16.
__device__ __forceinline__ void reduce_split_ml(const float2 (&ml)[4], float &M, float &W) {
  float m = fmaxf(fmaxf(ml[0].x, ml[1].x), fmaxf(ml[2].x, ml[3].x));
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  float l = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (ml[k].x != -INFINITY) l = fmaf(ml[k].y, __builtin_amdgcn_exp2f(ml[k].x - m), l);
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) l += __shfl_xor(l, o);
  M = m;
  W = l;
}

// Output rows, 256 threads: group q = tid / 32 takes splits q, q + 8, ...,
// q + 56 and lane c4 = tid % 32 the columns 4 c4 .. 4 c4 + 3.  ok false: none.
__device__ __forceinline__ void load_split_row(const AttnArgs &a, size_t rows, size_t li, int q, int c4, bool ok,
                                               float (&ms)[8], float4 (&po)[8]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int sp = q + 8 * k;
    ms[k] = -INFINITY;
    po[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (ok && sp < a.nsplit) {
      const size_t pr = sp * rows + li;
      ms[k] = a.part_ml[2 * pr];
      po[k] = *reinterpret_cast<const float4 *>(a.part + pr * MERGE_D + 4 * c4);
    }
  }
}

// Output row li from the partials load_split_row gave the 256 merging
// threads (merger true for them; M, W of the row from reduce_split_ml, L its
// normaliser): each group weights its splits by 2^(m_s - M), the eight
// group sums meet in red_o, and threads 0..31 add them in group order and
// write the bf16 row and its normalisers.  Contains a block barrier: every
// thread of the workgroup calls it.
__device__ __forceinline__ void merge_split_row(const AttnArgs &a, size_t li, float M, float W, float L, int q,
                                                int c4, bool merger, const float (&ms)[8], const float4 (&po)[8],
                                                float4 (*red_o)[32]) {
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (ms[k] == -INFINITY) continue;
    const float w = __builtin_amdgcn_exp2f(ms[k] - M);
    acc.x = fmaf(po[k].x, w, acc.x);
    acc.y = fmaf(po[k].y, w, acc.y);
    acc.z = fmaf(po[k].z, w, acc.z);
    acc.w = fmaf(po[k].w, w, acc.w);
  }
  if (merger) red_o[q][c4] = acc;
  __syncthreads();
  if (threadIdx.x < 32) {
    float4 t = red_o[0][c4];
#pragma unroll
    for (int k = 1; k < 8; ++k) {
      const float4 u = red_o[k][c4];
      t.x += u.x;
      t.y += u.y;
      t.z += u.z;
      t.w += u.w;
    }
    const float inv = 1.f / W;
    const uint32_t lo = static_cast<uint32_t>(f32_to_bf16(t.x * inv)) |
                        (static_cast<uint32_t>(f32_to_bf16(t.y * inv)) << 16);
    const uint32_t hi = static_cast<uint32_t>(f32_to_bf16(t.z * inv)) |
                        (static_cast<uint32_t>(f32_to_bf16(t.w * inv)) << 16);
    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + li * MERGE_D + 4 * c4) = make_uint2(lo, hi);
    if (c4 == 0) {
      a.lse2[li] = L;
      if (a.lse_nat) a.lse_nat[li] = L * 0.69314718055994530942f;
    }
  }
}

// Summed weight of one key over the group's R (<= LOGIT_ROWS_MAX) rows,
// Kahan-compensated in row order: x(r) gives the stored logit of row r, xs
// brings it to log2 units, Ls[r] is the row's normaliser, and visible(r)
// says whether row r sees the key.  Unrolled, so x may index registers.
template <typename X, typename V>
__device__ __forceinline__ float key_weight_sum(int R, X &&x, V &&visible, float xs, const float *Ls) {
  float acc = 0.f, comp = 0.f;
#pragma unroll
  for (int r = 0; r < LOGIT_ROWS_MAX; ++r) {
    if (r < R && visible(r)) {
      const float p = __builtin_amdgcn_exp2f(fmaf(x(r), xs, -Ls[r]));
      const float y = p - comp;
      const float s2 = acc + y;
      comp = (s2 - acc) - y;
      acc = s2;
    }
  }
  return acc;
}

}  // namespace h2o
