// LDS tile helpers shared by the bf16 matrix-core attention kernels for
// gfx950 (native and quantised caches, head dimension 128): operand types,
// buffer-resource LDS DMA, the XOR swizzles of K/Q and V tiles, and transpose
// reads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_util.hpp"

namespace h2o {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int D = 128;
constexpr int ROW_BYTES = D * 2;    // 256
constexpr int TILE_BYTES = 64 * ROW_BYTES;  // 64 rows x 128 bf16 = 16 KB
constexpr float RESCALE_SLACK = 8.f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Raw buffer resource over `bytes` bytes at `base` (gfx9 descriptor word 3:
// 32-bit data format, no swizzle).  Lanes whose offset is past `bytes` read 0.
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(bytes), 0x00020000);
}

// LDS DMA: lane l's `size` bytes from base + voff + soff land at lds_segment + size*l.
__device__ __forceinline__ void dma16(rsrc_t r, uint32_t voff, uint32_t soff, char *lds_segment) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(lds_segment), 16, voff, soff, 0, 0);
}

__device__ __forceinline__ void dma4(rsrc_t r, uint32_t voff, uint32_t soff, char *lds_segment) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(lds_segment), 4, voff, soff, 0, 0);
}

__device__ __forceinline__ void wait_dma_and_sync() {
  __builtin_amdgcn_s_waitcnt(0);  // this wavefront's loads (incl. LDS DMA) are done
  __syncthreads();                // ... and everybody else's
}

// K / Q tile: chunk c of row r at r*256 + 16*(c ^ (r & 15)) -- 16 consecutive
// rows read at one chunk index touch 16 distinct 16-byte bank groups.
__device__ __forceinline__ int kq_off(int row, int chunk) {
  return row * ROW_BYTES + ((chunk ^ (row & 15)) << 4);
}
__device__ __forceinline__ int kq_chunk_at(int row, int pos) { return pos ^ (row & 15); }

// V tile: chunk c of row r at r*256 + 16*(c ^ 4*(r & 3)) -- the 4 rows x 4
// chunks a transpose read touches per half-wave land on 16 distinct groups.
__device__ __forceinline__ int v_off(int row, int chunk) {
  return row * ROW_BYTES + ((chunk ^ ((row & 3) << 2)) << 4);
}
__device__ __forceinline__ int v_chunk_at(int row, int pos) { return pos ^ ((row & 3) << 2); }

// V tile the 8/4-bit passes widen into: chunk c of row r at
// r*256 + 16*(c ^ 5*(r & 3)).  Over 4 aligned rows (j = r & 3) a chunk
// 4b + i lands at 4(b ^ j) + (i ^ j), so the same transpose reads and also
// the stores of widened rows (4 aligned rows x chunks 4q + i, q = 0..3) meet
// 16 distinct groups; with 4*(r & 3) those stores met 4 lanes per bank.
__device__ __forceinline__ int vq_off(int row, int chunk) {
  return row * ROW_BYTES + ((chunk ^ (5 * (row & 3))) << 4);
}

__device__ __forceinline__ bf16x8 lds16(const char *p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(p));
}

__device__ __forceinline__ i16x4 lds_tr(const char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
}

// Tiles the backward reads both row-wise (16 rows at one chunk index) and
// transposed (4 aligned rows x 4 aligned chunks per half-wave): chunk c of
// row r at r*256 + 16*(c ^ g(r)), g(r) = 4*(r & 3) + ((r >> 2) & 3).  g is a
// bijection of r & 15, so a row-wise read meets 16 distinct 16-byte groups;
// over 4 aligned rows (r >> 2) & 3 is fixed and 4*(r & 3) moves the 4
// aligned chunks to 4 distinct quarters, so a transpose read meets all 16
// groups too (the K/Q swizzle put those 4 x 4 chunks on 4 groups: a 4-way
// bank conflict).
__device__ __forceinline__ int bt_swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
__device__ __forceinline__ int bt_off(int row, int chunk) { return row * ROW_BYTES + ((chunk ^ bt_swz(row)) << 4); }
__device__ __forceinline__ int bt_chunk_at(int row, int pos) { return pos ^ bt_swz(row); }

// Transpose read of a bt-swizzled tile: for lane l the 8 rows
// 16*ks + 8*(l/32) + 0..7 at column 32*blk + l%32 (the A operand of a product
// whose K dimension runs along the tile's rows).
__device__ __forceinline__ bf16x8 tr_operand(const char *tb, int ks, int blk, int lane) {
  const int grp16 = lane >> 4, i16 = lane & 15;
  const int row = 16 * ks + 8 * (grp16 >> 1) + (i16 >> 2);
  const int col = 32 * blk + 16 * (grp16 & 1) + 4 * (i16 & 3);
  const bf16x4 lo = __builtin_bit_cast(bf16x4, lds_tr(tb + bt_off(row, col >> 3) + 2 * (col & 7)));
  const bf16x4 hi = __builtin_bit_cast(bf16x4, lds_tr(tb + bt_off(row + 4, col >> 3) + 2 * (col & 7)));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ int perm_key(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

__device__ __forceinline__ uint32_t pack_bf16_rne(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// The same rounding (to nearest even) by one v_cvt_pk_bf16_f32, for MFMA
// operands inside tile loops; pack_bf16_rne's NaN test compiles to a branch.
__device__ __forceinline__ uint32_t pack_bf16_hw(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

}  // namespace
}  // namespace h2o
