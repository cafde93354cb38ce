// One wavefront quantises one key or value row of the chunk into a slot of
// an 8-bit or 4-bit cache.  Shared by the write kernel and by the selection's
// pick kernel, which writes the rows itself for short chunks, so the codes
// are the same bit for bit on both paths.
//
// The pages name 8-bit and 4-bit buffers without a scheme (aimodeling
// article; "Learning how to Forget", §2); the scheme here is, per slot and KV
// head, with IEEE fp32 operations and round-to-nearest-even:
//   int8: a = max|x|; s = fp16(a/127); c = clamp(rne(x/s), -127, 127)
//   int4: z = fp16(min x); s = fp16((max - min)/15); c = clamp(rne((x - z)/s), 0, 15)
//   s == 0 -> all codes 0; element 2k of an int4 row in the low nibble of byte k.
#pragma once

#include "device_util.hpp"
#include "h2o_internal.hpp"

namespace h2o {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o));
  return v;
}

// Chunk row rr (= group * T + t) of K (isv false) or V into cache row
// dst_row (= group * C + slot).  Lane l handles elements 2l and 2l + 1
// (D <= 128); every lane of the wavefront must call it.
template <int DT, int FMT>
__device__ __forceinline__ void quantize_row(const KvWriteArgs &a, size_t rr, size_t dst_row, bool isv, int lane) {
  const void *src = isv ? a.vn : a.kn;
  const bool has = 2 * lane < a.D;
  const float x0 = has ? load_elem<DT>(src, rr * a.D + 2 * lane) : 0.f;
  const float x1 = has ? load_elem<DT>(src, rr * a.D + 2 * lane + 1) : 0.f;
  if constexpr (FMT == FMT_INT8) {
    const float amax = wave_max(has ? fmaxf(fabsf(x0), fabsf(x1)) : 0.f);
    const uint16_t s16 = f32_to_f16(amax / 127.0f);
    const float s = f16_to_f32(s16);
    int c0 = 0, c1 = 0;
    if (s != 0.f) {
      c0 = static_cast<int>(fminf(fmaxf(rintf(x0 / s), -127.f), 127.f));
      c1 = static_cast<int>(fminf(fmaxf(rintf(x1 / s), -127.f), 127.f));
    }
    int8_t *codes = static_cast<int8_t *>(isv ? a.vc : a.kc);
    if (has) {
      const uint16_t packed = static_cast<uint16_t>((c0 & 0xff) | ((c1 & 0xff) << 8));
      *reinterpret_cast<uint16_t *>(codes + dst_row * a.D + 2 * lane) = packed;
    }
    if (lane == 0) (isv ? a.vs : a.ks)[dst_row] = s16;
  } else {
    const float lo = wave_min(has ? fminf(x0, x1) : INFINITY);
    const float hi = wave_max(has ? fmaxf(x0, x1) : -INFINITY);
    const uint16_t z16 = f32_to_f16(lo);
    const float z = f16_to_f32(z16);
    const float span = hi - lo;
    const uint16_t s16 = f32_to_f16(span / 15.0f);
    const float s = f16_to_f32(s16);
    int c0 = 0, c1 = 0;
    if (s != 0.f) {
      c0 = static_cast<int>(fminf(fmaxf(rintf((x0 - z) / s), 0.f), 15.f));
      c1 = static_cast<int>(fminf(fmaxf(rintf((x1 - z) / s), 0.f), 15.f));
    }
    uint8_t *codes = static_cast<uint8_t *>(isv ? a.vc : a.kc);
    if (has) codes[dst_row * (a.D / 2) + lane] = static_cast<uint8_t>(c0 | (c1 << 4));
    if (lane == 0) {
      (isv ? a.vs : a.ks)[dst_row] = s16;
      (isv ? a.vz : a.kz)[dst_row] = z16;
    }
  }
}

}  // namespace h2o
