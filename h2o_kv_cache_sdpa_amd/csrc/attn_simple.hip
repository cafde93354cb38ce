// Portable fp32 VALU attention passes (no matrix cores).  Used for the fp32
// dtype, where the chunk step must match exact attention to 1e-5 absolute,
// and for every cache format.  One thread owns one packed query row (pass A)
// or one key (pass B).
//
// Pass A: online-softmax attention ("Learning how to Forget", §A.7: softmax of
//   mask(scale Q K^T) applied to V) -> out and the log2-domain normaliser.
// Pass B: the weights exp2(x - L) recomputed with the final normaliser and
//   summed over all query rows of the KV group -> wsum (§3.1.1, §A.7).
// Query rows of a KV group are packed as r = i*q_g + hh (chunk position i,
// head hh of the group); cache slots j < n_occ are all visible, chunk key t is
// visible to row r iff t <= i (§A.1 mask with the chunk written after it
// attends).

#include "device_util.hpp"
#include "h2o_internal.hpp"

namespace h2o {
namespace {

constexpr int ROWS_A = 64;  // query rows per block in pass A
constexpr int KT = 32;      // keys per LDS tile
constexpr int KEYS_B = 64;  // keys per block in pass B
constexpr int RT = 32;      // query rows per LDS tile in pass B

template <int DT, int FMT>
__device__ __forceinline__ float key_value(const AttnArgs &a, const void *cache, const uint16_t *sc,
                                           const uint16_t *zr, const void *newbuf, int grp, int j,
                                           int d) {
  if (j < a.n_occ) {
    return cache_elem<DT, FMT>(cache, sc, zr, static_cast<size_t>(grp) * a.C + j, d, a.D);
  }
  const int t = j - a.n_occ;
  return load_elem<DT>(newbuf, (static_cast<size_t>(grp) * a.T + t) * a.D + d);
}

template <int DT, int FMT, int D>
__global__ __launch_bounds__(ROWS_A) void attn_a_simple(AttnArgs a) {
  __shared__ float Qs[ROWS_A][D + 1];
  __shared__ float Ks[KT][D];
  __shared__ float Vs[KT][D];
  const int grp = blockIdx.y;
  const int g = grp % a.Hkv;
  const int b = grp / a.Hkv;
  const int rows = a.qg * a.T;
  const int r0 = blockIdx.x * ROWS_A;
  const int tid = threadIdx.x;
  const int r = r0 + tid;
  const bool active = r < rows;
  const int i = active ? r / a.qg : 0;
  const int h = g * a.qg + (active ? r % a.qg : 0);

  for (int e = tid; e < ROWS_A * D; e += ROWS_A) {
    const int rr = e / D, d = e % D;
    const int rw = r0 + rr;
    float v = 0.f;
    if (rw < rows) {
      const int ii = rw / a.qg, hh = g * a.qg + rw % a.qg;
      v = load_elem<DT>(a.q, ((static_cast<size_t>(b) * a.Hq + hh) * a.T + ii) * D + d);
    }
    Qs[rr][d] = v;
  }

  const int last_row = min(rows, r0 + ROWS_A) - 1;
  const int key_end = a.n_occ + last_row / a.qg + 1;  // keys any row of the block sees

  float m = -INFINITY, l = 0.f;
  float o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) o[d] = 0.f;

  for (int j0 = 0; j0 < key_end; j0 += KT) {
    __syncthreads();
    for (int e = tid; e < KT * D; e += ROWS_A) {
      const int kk = e / D, d = e % D;
      const int j = j0 + kk;
      float kv = 0.f, vv = 0.f;
      if (j < key_end) {
        kv = key_value<DT, FMT>(a, a.kc, a.ks, a.kz, a.kn, grp, j, d);
        vv = key_value<DT, FMT>(a, a.vc, a.vs, a.vz, a.vn, grp, j, d);
      }
      Ks[kk][d] = kv;
      Vs[kk][d] = vv;
    }
    __syncthreads();
    const int kend = min(KT, key_end - j0);
    for (int kk = 0; kk < kend; ++kk) {
      const int j = j0 + kk;
      const bool visible = active && (j < a.n_occ || (j - a.n_occ) <= i);
      if (!visible) continue;
      float dot = 0.f;
#pragma unroll 16
      for (int d = 0; d < D; ++d) dot = fmaf(Qs[tid][d], Ks[kk][d], dot);
      const float x = dot * a.sl2;
      if (x > m) {
        const float alpha = exp2f(m - x);  // 0 when m = -inf
        l = l * alpha + 1.f;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] = fmaf(o[d], alpha, Vs[kk][d]);
        m = x;
      } else {
        const float p = exp2f(x - m);
        l += p;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] = fmaf(p, Vs[kk][d], o[d]);
      }
    }
  }
  if (!active) return;
  const float inv = 1.f / l;
  const size_t orow = ((static_cast<size_t>(b) * a.Hq + h) * a.T + i) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const float v = o[d] * inv;
    if constexpr (DT == 0) {
      reinterpret_cast<float *>(a.out)[orow + d] = v;
    } else {
      reinterpret_cast<uint16_t *>(a.out)[orow + d] = f32_to_bf16(v);
    }
  }
  const float L = m + log2f(l);
  const size_t li = (static_cast<size_t>(b) * a.Hq + h) * a.T + i;
  a.lse2[li] = L;
  if (a.lse_nat) a.lse_nat[li] = L * 0.69314718055994530942f;
}

template <int DT, int FMT, int D>
__global__ __launch_bounds__(KEYS_B) void attn_b_simple(AttnArgs a) {
  __shared__ float Qs[RT][D];
  __shared__ float Ls[RT];
  const int grp = blockIdx.y;
  const int g = grp % a.Hkv;
  const int b = grp / a.Hkv;
  const int rows = a.qg * a.T;
  const int n_keys = a.n_occ + a.T;
  const int tid = threadIdx.x;
  const int j0 = blockIdx.x * KEYS_B;
  const int j = j0 + tid;
  const bool active = j < n_keys;

  float kv[D];
#pragma unroll
  for (int d = 0; d < D; ++d)
    kv[d] = active ? key_value<DT, FMT>(a, a.kc, a.ks, a.kz, a.kn, grp, j, d) : 0.f;
  const int tnew = j - a.n_occ;  // >= 0 for a chunk key

  // rows before the first chunk key of the block cannot see any key of it
  const int first_new = max(0, j0 - a.n_occ);
  const int row_begin = (j0 < a.n_occ) ? 0 : first_new * a.qg;

  float acc = 0.f, comp = 0.f;  // compensated (Kahan) running sum
  for (int rb = row_begin - row_begin % RT; rb < rows; rb += RT) {
    __syncthreads();
    for (int e = tid; e < RT * D; e += KEYS_B) {
      const int rr = e / D, d = e % D;
      const int rw = rb + rr;
      float v = 0.f;
      if (rw < rows) {
        const int ii = rw / a.qg, hh = g * a.qg + rw % a.qg;
        v = load_elem<DT>(a.q, ((static_cast<size_t>(b) * a.Hq + hh) * a.T + ii) * D + d);
      }
      Qs[rr][d] = v;
    }
    if (tid < RT) {
      const int rw = rb + tid;
      float L = 0.f;
      if (rw < rows) {
        const int ii = rw / a.qg, hh = g * a.qg + rw % a.qg;
        L = a.lse2[(static_cast<size_t>(b) * a.Hq + hh) * a.T + ii];
      }
      Ls[tid] = L;
    }
    __syncthreads();
    const int rend = min(RT, rows - rb);
    float part = 0.f;
    for (int rr = 0; rr < rend; ++rr) {
      const int i = (rb + rr) / a.qg;
      const bool visible = active && (tnew < 0 || tnew <= i);
      if (!visible) continue;
      float dot = 0.f;
#pragma unroll 16
      for (int d = 0; d < D; ++d) dot = fmaf(Qs[rr][d], kv[d], dot);
      part += exp2f(fmaf(dot, a.sl2, -Ls[rr]));
    }
    const float y = part - comp;
    const float t = acc + y;
    comp = (t - acc) - y;
    acc = t;
  }
  if (active) a.wsum[static_cast<size_t>(grp) * n_keys + j] = acc;
}

template <int DT, int FMT, int D>
hipError_t launch_simple_t(const AttnArgs &a, hipStream_t s) {
  const int groups = a.B * a.Hkv;
  const int rows = a.qg * a.T;
  dim3 ga((rows + ROWS_A - 1) / ROWS_A, groups);
  {
    KernelTimer timer(H2O_K_ATTN_A, s);
    hipLaunchKernelGGL((attn_a_simple<DT, FMT, D>), ga, dim3(ROWS_A), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.wsum) return e;
  const int n_keys = a.n_occ + a.T;
  dim3 gb((n_keys + KEYS_B - 1) / KEYS_B, groups);
  {
    KernelTimer timer(H2O_K_ATTN_B, s);
    hipLaunchKernelGGL((attn_b_simple<DT, FMT, D>), gb, dim3(KEYS_B), 0, s, a);
  }
  return hipGetLastError();
}

template <int DT, int FMT>
hipError_t launch_simple_d(const AttnArgs &a, hipStream_t s) {
  if (a.D == 64) return launch_simple_t<DT, FMT, 64>(a, s);
  return launch_simple_t<DT, FMT, 128>(a, s);
}

template <int DT>
hipError_t launch_simple_f(const AttnArgs &a, hipStream_t s) {
  switch (a.cache_fmt) {
    case FMT_INT8: return launch_simple_d<DT, FMT_INT8>(a, s);
    case FMT_INT4: return launch_simple_d<DT, FMT_INT4>(a, s);
    default: return launch_simple_d<DT, FMT_NATIVE>(a, s);
  }
}

}  // namespace

hipError_t launch_attn_simple(const AttnArgs &a, hipStream_t s) {
  if (a.dtype == DT_F32) return launch_simple_f<DT_F32>(a, s);
  return launch_simple_f<DT_BF16>(a, s);
}

}  // namespace h2o
