// Codes of 8-bit and 4-bit cache rows widened to bf16 MFMA operands, shared by
// the quantised attention passes (head dimension 128).  Codes are integers,
// exact in bf16: an 8-bit cache stores x = c s per slot, a 4-bit cache
// x = c s + z with c in 0..15 (two codes per byte, element 2i in the low
// nibble of byte i).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "h2o_internal.hpp"

namespace h2o {
namespace {

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

}  // namespace
}  // namespace h2o
