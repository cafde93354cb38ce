// Backward of the chunk attention, dQ ("Learning how to Forget", §3.2): see
// attn_bwd.hip for the formulas.  bwd_dq: 128 query rows per workgroup
// (4 waves x 32; 256 rows, 8 waves, for the row terms), K and V tiles of 64 keys moved HBM -> LDS by buffer-load
// DMA, double-buffered.  S^T = K Q^T and dP^T = V dO^T on the matrix cores
// with Q and dO held in registers; dS in registers becomes the B operand of
// dQ^T += K^T dS^T, the K^T operand read from the row-major K tile by
// ds_read_b64_tr_b16 (as V^T in pass A).
//
// The same kernel with ROWTERM = true runs first and forms each row's term
// D_r = sum_j P_rj dP_rj from the recomputed fp32 P and dP of every visible
// key (plus L2_r = lse_r log2 e), so that dS = P (dP - D) is taken against
// the row term of this P and dP.  (D_r also equals <dO_r, O_r>, but the
// stored output is bf16, and the rounding of O shifts every dS_rj of the
// row by P_rj times the same error, which becomes visible wherever
// dP_rj - D_r cancels.)
//
// This file is built with the VGPR form of the MFMAs: the kernel runs one
// wavefront per SIMD with more than 256 registers, and otherwise its S / dP
// results would sit in accumulation registers and be copied out before every
// exponential.

#include "device_util.hpp"
#include "h2o_internal.hpp"
#include "tile_util.hpp"

namespace h2o {
namespace {

constexpr float LOG2E = 1.4426950408889634074f;
constexpr int SG_VALU = 0x002, SG_MFMA = 0x008;  // __builtin_amdgcn_sched_group_barrier masks

// dQ (ROWTERM = false) or the row terms L2, D (ROWTERM = true): 32 packed
// query rows (r = i * q_g + h) per wavefront, NW wavefronts per block, keys
// streamed.  dQ needs more than 256 registers (4 wavefronts, one per SIMD);
// the row terms fit two per SIMD, so 8 wavefronts share each K / V tile.
template <bool ROWTERM, int NW>
__global__ __launch_bounds__(64 * NW, 1) void bwd_dq(BwdArgs a) {
  constexpr int ROWS = 32 * NW, SPW = 16 / NW;  // rows per block, 1 KB tile segments per wavefront
  __shared__ __attribute__((aligned(1024))) char kb0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char kb1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vb0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vb1[TILE_BYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, hl = lane >> 5;
  const int R = a.qg * a.T;
  const int tiles_per_grp = (R + ROWS - 1) / ROWS;
  const int wi = xcd_remap(blockIdx.x, gridDim.x);
  // Row blocks go out last first: under the causal mask the last rows see the
  // most keys, and starting the longest blocks first evens out the tail.
  const int grp = wi / tiles_per_grp, rt = tiles_per_grp - 1 - wi % tiles_per_grp;
  const int g = grp % a.Hkv, b = grp / a.Hkv;
  const int row0 = rt * ROWS;
  const int my_row = row0 + wave * 32 + n;
  const bool row_ok = my_row < R;
  const int i_q = row_ok ? my_row / a.qg : 0;
  // wave-uniform: all 32 rows exist; the smallest chunk position among them
  const bool wave_rows_ok = row0 + wave * 32 + 31 < R;
  const int wave_i_min = (row0 + wave * 32) / a.qg;
  const int h_q = g * a.qg + (row_ok ? my_row % a.qg : 0);
  const size_t li = (static_cast<size_t>(b) * a.Hq + h_q) * a.T + i_q;
  const int n_occ = a.n_occ;
  const float sl2 = a.sl2;

  // Q and dO rows: B operands of S^T = K Q^T and dP^T = V dO^T
  bf16x8 qf[8], gf[8];
  {
    const uint16_t *qrow = static_cast<const uint16_t *>(a.q) + li * D;
    const uint16_t *grow = static_cast<const uint16_t *>(a.dout) + li * D;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      uint4 vq = make_uint4(0, 0, 0, 0), vg = make_uint4(0, 0, 0, 0);
      if (row_ok) {
        vq = *reinterpret_cast<const uint4 *>(qrow + 16 * st + 8 * hl);
        vg = *reinterpret_cast<const uint4 *>(grow + 16 * st + 8 * hl);
      }
      qf[st] = __builtin_bit_cast(bf16x8, vq);
      gf[st] = __builtin_bit_cast(bf16x8, vg);
    }
  }
  const float Lr = !row_ok ? 0.f : ROWTERM ? a.lse[li] * LOG2E : a.l2[li];
  const float Dr = (row_ok && !ROWTERM) ? a.dd[li] : 0.f;
  float d_acc = 0.f;  // ROWTERM: sum of P dP over the keys so far

  const int last_row = min(R, row0 + ROWS) - 1;
  const int key_end = n_occ + last_row / a.qg + 1;
  const int ntiles = (key_end + 63) / 64;
  const size_t cache_row0 = static_cast<size_t>(grp) * a.C;
  const size_t new_row0 = static_cast<size_t>(grp) * a.T;
  const rsrc_t kc_rs = make_rsrc(static_cast<const char *>(a.kc) + cache_row0 * ROW_BYTES, n_occ * ROW_BYTES);
  const rsrc_t vc_rs = make_rsrc(static_cast<const char *>(a.vc) + cache_row0 * ROW_BYTES, n_occ * ROW_BYTES);
  const rsrc_t kn_rs = make_rsrc(static_cast<const char *>(a.kn) + new_row0 * ROW_BYTES, a.T * ROW_BYTES);
  const rsrc_t vn_rs = make_rsrc(static_cast<const char *>(a.vn) + new_row0 * ROW_BYTES, a.T * ROW_BYTES);
  // both tiles in the bt swizzle: read row-wise for S^T / dP^T and (K) transposed for dQ
  auto lane_off = [&](int q) -> uint32_t {
    const int row = (wave * SPW + q) * 4 + (lane >> 4);
    return static_cast<uint32_t>(row * ROW_BYTES + 16 * bt_chunk_at(row, lane & 15));
  };
  auto issue_tile = [&](int tile, char *dst, rsrc_t crs, rsrc_t nrs) {
    const int j0 = tile * 64;
    if (j0 + 64 <= n_occ) {
#pragma unroll
      for (int q = 0; q < SPW; ++q) dma16(crs, lane_off(q), j0 * ROW_BYTES, dst + (wave * SPW + q) * 1024);
    } else {
      const int dt = j0 - n_occ;  // chunk index of the tile's first row, may be < 0
#pragma unroll
      for (int q = 0; q < SPW; ++q) {
        const int row = (wave * SPW + q) * 4 + (lane >> 4);
        const uint32_t lo = lane_off(q);
        if (dt + row >= 0) {
          dma16(nrs, lo + dt * ROW_BYTES, 0, dst + (wave * SPW + q) * 1024);
        } else {
          dma16(crs, lo + j0 * ROW_BYTES, 0, dst + (wave * SPW + q) * 1024);
        }
      }
    }
  };

  const int prow = perm_key(n);
  f32x16 dq[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) dq[k] = f32x16{};

  // Row terms of one 64-key tile: the S / dP MFMAs of the second 32-key half
  // run beside the exponentials of the first (the terms need no dQ product,
  // so both halves' results fit in registers at once).
  auto rowterm_tile = [&](int t, const char *kb, const char *vb) __attribute__((always_inline)) {
    f32x16 s0 = f32x16{}, p0 = f32x16{}, s1 = f32x16{}, p1 = f32x16{};
    float part = 0.f;
    // wave-uniform: every row of the wave exists and sees every key of the half
    const bool full0 = wave_rows_ok && t * 64 + 31 - n_occ <= wave_i_min;
    const bool full1 = wave_rows_ok && t * 64 + 63 - n_occ <= wave_i_min;
    auto term = [&](bool full, int k0, float sv, float dpv, int r) {
      const int ja = t * 64 + k0 + 16 * (r >> 3) + 8 * hl + (r & 7) - n_occ;  // chunk index
      const bool vis = full || (row_ok && ja <= i_q);
      const float pp = vis ? __builtin_amdgcn_exp2f(fmaf(sv, sl2, -Lr)) : 0.f;
      part = fmaf(pp, dpv, part);
    };
    auto chain = [&](int k0, f32x16 &sacc, f32x16 &pacc, bool overlap) {
      const int kr = k0 + prow;
      bf16x8 ka = lds16(kb + bt_off(kr, hl)), va = lds16(vb + bt_off(kr, hl));
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        bf16x8 nk = ka, nv = va;
        if (st < 7) {
          nk = lds16(kb + bt_off(kr, 2 * st + 2 + hl));
          nv = lds16(vb + bt_off(kr, 2 * st + 2 + hl));
        }
        __builtin_amdgcn_sched_barrier(0);
        sacc = mfma32(ka, qf[st], sacc);
        pacc = mfma32(va, gf[st], pacc);
        ka = nk;
        va = nv;
        if (overlap) {  // two of the first half's 16 terms per step
          term(full0, 0, s0[2 * st], p0[2 * st], 2 * st);
          term(full0, 0, s0[2 * st + 1], p0[2 * st + 1], 2 * st + 1);
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(SG_VALU, 3, 0);
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(SG_VALU, 3, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    chain(0, s0, p0, false);
    chain(32, s1, p1, true);
#pragma unroll
    for (int r = 0; r < 16; ++r) term(full1, 32, s1[r], p1[r], r);
    d_acc += part;
  };

  // One 64-key tile in two halves of 32 keys (keeps one S / dP pair live).
  auto compute = [&](int t, const char *kb, const char *vb) __attribute__((always_inline)) {
    if constexpr (ROWTERM) {
      rowterm_tile(t, kb, vb);
      return;
    }
#pragma unroll 1
    for (int half = 0; half < 2; ++half) {
      const int kr = 32 * half + prow;  // K / V row of the lane's operand
      f32x16 s0 = f32x16{}, p0 = f32x16{};
      // operands one step ahead of their MFMAs; the barriers keep the compiler
      // from hoisting every step's reads (and their registers) to the top
      bf16x8 k0 = lds16(kb + bt_off(kr, hl)), v0 = lds16(vb + bt_off(kr, hl));
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        bf16x8 nk0 = k0, nv0 = v0;
        if (st < 7) {
          nk0 = lds16(kb + bt_off(kr, 2 * st + 2 + hl));
          nv0 = lds16(vb + bt_off(kr, 2 * st + 2 + hl));
        }
        __builtin_amdgcn_sched_barrier(0);
        s0 = mfma32(k0, qf[st], s0);
        p0 = mfma32(v0, gf[st], p0);
        k0 = nk0;
        v0 = nv0;
        __builtin_amdgcn_sched_barrier(0);
      }
      // register r: key t*64 + 32*half + 16*(r/8) + 8*hl + r%8 of the lane's row
      // wave-uniform: every row of the wave exists and sees every key of the half
      const bool half_full = wave_rows_ok && t * 64 + 32 * half + 31 - n_occ <= wave_i_min;
      bf16x8 dsb[2];
      if (half_full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pp = __builtin_amdgcn_exp2f(fmaf(s0[r], sl2, -Lr));
          dsb[r >> 3][r & 7] = static_cast<__bf16>(pp * (p0[r] - Dr));
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ja = t * 64 + 32 * half + 16 * (r >> 3) + 8 * hl + (r & 7) - n_occ;  // chunk index
          const bool vis = row_ok && ja <= i_q;
          const float pp = vis ? __builtin_amdgcn_exp2f(fmaf(s0[r], sl2, -Lr)) : 0.f;
          dsb[r >> 3][r & 7] = static_cast<__bf16>(pp * (p0[r] - Dr));
        }
      }
      // dQ^T += K^T dS^T over the half's keys (k-steps 2*half, 2*half + 1)
      bf16x8 kt = tr_operand(kb, 2 * half, 0, lane);
#pragma unroll
      for (int step = 0; step < 8; ++step) {
        const int ks = step >> 2, blk = step & 3;
        bf16x8 nkt = kt;
        if (step < 7) nkt = tr_operand(kb, 2 * half + ((step + 1) >> 2), (step + 1) & 3, lane);
        __builtin_amdgcn_sched_barrier(0);
        dq[blk] = mfma32(kt, dsb[ks], dq[blk]);
        kt = nkt;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  if (ntiles > 0) {
    issue_tile(0, kb0, kc_rs, kn_rs);
    issue_tile(0, vb0, vc_rs, vn_rs);
  }
  for (int t = 0; t < ntiles; t += 2) {
    wait_dma_and_sync();  // tile t in kb0/vb0; everybody done with kb1/vb1
    if (t + 1 < ntiles) {
      issue_tile(t + 1, kb1, kc_rs, kn_rs);
      issue_tile(t + 1, vb1, vc_rs, vn_rs);
    }
    compute(t, kb0, vb0);
    if (t + 1 >= ntiles) break;
    wait_dma_and_sync();  // tile t+1 in kb1/vb1; everybody done with kb0/vb0
    if (t + 2 < ntiles) {
      issue_tile(t + 2, kb0, kc_rs, kn_rs);
      issue_tile(t + 2, vb0, vc_rs, vn_rs);
    }
    compute(t + 1, kb1, vb1);
  }

  if constexpr (ROWTERM) {
    const float d_row = d_acc + __shfl_xor(d_acc, 32);
    if (row_ok && hl == 0) {
      a.dd[li] = d_row;
      a.l2[li] = Lr;
    }
    return;
  }
  if (!row_ok) return;
  float *dst = a.dq + li * D;
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int d = 32 * blk + 8 * a4 + 4 * hl;
      *reinterpret_cast<float4 *>(dst + d) =
          make_float4(dq[blk][4 * a4] * a.scale, dq[blk][4 * a4 + 1] * a.scale,
                      dq[blk][4 * a4 + 2] * a.scale, dq[blk][4 * a4 + 3] * a.scale);
    }
  }
}

}  // namespace

hipError_t launch_bwd_dq(const BwdArgs &a, hipStream_t s) {
  const int groups = a.B * a.Hkv;
  const int R = a.qg * a.T;
  {
    KernelTimer timer(H2O_K_BWD_ROWS, s);
    hipLaunchKernelGGL((bwd_dq<true, 8>), dim3(groups * ((R + 255) / 256)), dim3(512), 0, s, a);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  KernelTimer timer(H2O_K_BWD_DQ, s);
  hipLaunchKernelGGL((bwd_dq<false, 4>), dim3(groups * ((R + 127) / 128)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace h2o
