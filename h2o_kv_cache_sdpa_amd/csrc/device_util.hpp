// Small device helpers shared by the HIP kernels of libh2o.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h2o {

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bit pattern, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// fp32 -> fp16 bit pattern, round to nearest even (hardware conversion).
__device__ __forceinline__ uint16_t f32_to_f16(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

template <int DT>
__device__ __forceinline__ float load_elem(const void *p, size_t idx) {
  if constexpr (DT == 0) {
    return reinterpret_cast<const float *>(p)[idx];
  } else {
    return bf16_to_f32(reinterpret_cast<const uint16_t *>(p)[idx]);
  }
}

// Value of element d of cache row `row` (= grp*C + slot), dequantised to fp32.
template <int DT, int FMT>
__device__ __forceinline__ float cache_elem(const void *buf, const uint16_t *scale,
                                            const uint16_t *zero, size_t row, int d, int D) {
  if constexpr (FMT == 0) {
    return load_elem<DT>(buf, row * D + d);
  } else if constexpr (FMT == 1) {
    const int8_t c = reinterpret_cast<const int8_t *>(buf)[row * D + d];
    return static_cast<float>(c) * f16_to_f32(scale[row]);
  } else {
    const uint8_t byte = reinterpret_cast<const uint8_t *>(buf)[row * (D / 2) + d / 2];
    const int c = (d & 1) ? (byte >> 4) : (byte & 15);
    return fmaf(static_cast<float>(c), f16_to_f32(scale[row]), f16_to_f32(zero[row]));
  }
}

__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  // Blocks are dispatched round-robin over the 8 XCDs of an MI355X.  Remap so
  // that each XCD receives a contiguous range of work items (shared L2 lines).
  const int per = nblocks / 8;
  if (per * 8 != nblocks) return bid;
  return (bid % 8) * per + bid / 8;
}

}  // namespace h2o
