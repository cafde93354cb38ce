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

// Maximum of x over lanes l and l ^ 32.  v_permlane32_swap exchanges the
// wavefront's halves on the VALU; __shfl_xor would go through the LDS
// crossbar (ds_bpermute) and wait for every LDS access in flight.  With both
// operands x, the two results at lane l are x[l % 32] and x[32 + l % 32].
__device__ __forceinline__ float max_xor32(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

// Maximum of x over lanes l and l ^ 16 (v_permlane16_swap: rows of 16 lanes,
// odd rows of the first operand trade with even rows of the second; at lane
// l the two results are x of rows 2k and 2k + 1, k = l / 32).
__device__ __forceinline__ float max_xor16(float x) {
  const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

// v = min(v, u) for the 64-bit u made of the 32-bit halves lo, hi.
__device__ __forceinline__ void min_u64_halves(uint64_t &v, uint32_t lo, uint32_t hi) {
  const uint64_t u = (static_cast<uint64_t>(hi) << 32) | lo;
  v = u < v ? u : v;
}

// One DPP step of wave_min_u64: both halves take the lane move CTRL.
template <int CTRL>
__device__ __forceinline__ void dpp_min_u64(uint64_t &v) {
  const int lo = static_cast<int>(static_cast<uint32_t>(v));
  const int hi = static_cast<int>(static_cast<uint32_t>(v >> 32));
  min_u64_halves(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(lo, lo, CTRL, 0xf, 0xf, false)),
                 static_cast<uint32_t>(__builtin_amdgcn_update_dpp(hi, hi, CTRL, 0xf, 0xf, false)));
}

// Minimum of v over the wavefront, in every lane, without the LDS crossbar:
// DPP within rows of 16 lanes (neighbours in a quad, then the mirrored
// half-row and row, each pairing two groups that already agree), then
// v_permlane16_swap and v_permlane32_swap across rows.  Both 32-bit halves
// take the same lane moves, so every step compares whole 64-bit values.
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
  dpp_min_u64<0xb1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
  dpp_min_u64<0x4e>(v);   // quad_perm [2,3,0,1]: lane ^ 2
  dpp_min_u64<0x141>(v);  // row_half_mirror: quads 0 and 1 of each 8 lanes
  dpp_min_u64<0x140>(v);  // row_mirror: the two 8-lane halves of each row
  uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
  const auto l16 = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  const auto h16 = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  min_u64_halves(v, l16[0], h16[0]);
  min_u64_halves(v, l16[1], h16[1]);
  lo = static_cast<uint32_t>(v);
  hi = static_cast<uint32_t>(v >> 32);
  const auto l32 = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  const auto h32 = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  min_u64_halves(v, l32[0], h32[0]);
  min_u64_halves(v, l32[1], h32[1]);
  return v;
}

// Key tiles t_lo .. t_lo + count - 1 of split `split` of `nsplit` over
// `ntiles` tiles: the first ntiles % nsplit splits take one tile more, so no
// split holds more than one tile above another (count 0: an empty split).
__device__ __forceinline__ void split_tiles(int ntiles, int nsplit, int split, int &t_lo, int &count) {
  const int base = ntiles / nsplit, rem = ntiles % nsplit;
  t_lo = split * base + (split < rem ? split : rem);
  count = base + (split < rem ? 1 : 0);
}

__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  // Blocks are dispatched round-robin over the 8 XCDs of an MI355X.  Remap so
  // that each XCD receives a contiguous range of work items (shared L2 lines).
  const int per = nblocks / 8;
  if (per * 8 != nblocks) return bid;
  return (bid % 8) * per + bid / 8;
}

}  // namespace h2o
