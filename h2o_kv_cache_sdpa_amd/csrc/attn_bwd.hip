// Backward of the chunk attention for bf16 queries, a native bf16 cache and
// head dimension 128 ("Learning how to Forget", §3.2: gradients by reverse-mode
// differentiation through each chunk's SDPA call; §A.10: the attention
// interface that returns summed weights also has a backward).
//
// With P = softmax(mask(scale Q K^T)) as in the forward, per query row r of a
// KV group and key j of the group:
//   dP_rj = <dO_r, v_j>,  D_r = sum_j P_rj dP_rj (= <dO_r, O_r>),
//   dS_rj = P_rj (dP_rj - D_r),
//   dQ_r = scale sum_j dS_rj k_j,  dK_j = scale sum_r dS_rj q_r,  dV_j = sum_r P_rj dO_r.
// P is recomputed from the forward's row normalisers, exp2(s * scale * log2 e - L2_r).
//
// Three kernels, no atomics (every output element has one writer):
//  * bwd_dq<true> (attn_bwd_dq.hip): L2_r and D_r, the latter summed from the
//    recomputed fp32 P and dP over every visible key of the row;
//  * bwd_dq<false> (attn_bwd_dq.hip): 128 query rows per workgroup, K and V
//    tiles streamed (its own file: it is compiled with MFMA results in VGPRs);
//  * bwd_dkdv: 128 keys per workgroup (4 waves x 32) held in registers as
//    MFMA operands; 64-row blocks of Q and dO (and L2, D) stream through LDS,
//    double-buffered.  Q rows enter S = Q K^T in the same permuted order pass A
//    gives keys, so each half-wave holds runs of 8 consecutive rows of P and
//    dS: those are the A operands of dV += P^T dO and dK += dS^T Q directly,
//    and the dO / Q operands are transpose reads of the row blocks.
// P and dS enter the products rounded to bf16; all accumulation is fp32.

#include "device_util.hpp"
#include "h2o_internal.hpp"
#include "tile_util.hpp"

namespace h2o {
namespace {

// ---------------------------------------------------------------------------
// dK, dV: 128 keys per block (4 waves x 32), query rows streamed in blocks of 64
// ---------------------------------------------------------------------------
constexpr int BK_KEYS = 128;
constexpr int BR_ROWS = 64;
constexpr int RBLK_BYTES = BR_ROWS * ROW_BYTES;  // 16 KB

__global__ __launch_bounds__(256, 1) void bwd_dkdv(BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) char qb0[RBLK_BYTES];
  __shared__ __attribute__((aligned(1024))) char qb1[RBLK_BYTES];
  __shared__ __attribute__((aligned(1024))) char gb0[RBLK_BYTES];
  __shared__ __attribute__((aligned(1024))) char gb1[RBLK_BYTES];
  __shared__ __attribute__((aligned(256))) float lb0[BR_ROWS];
  __shared__ __attribute__((aligned(256))) float lb1[BR_ROWS];
  __shared__ __attribute__((aligned(256))) float db0[BR_ROWS];
  __shared__ __attribute__((aligned(256))) float db1[BR_ROWS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, hl = lane >> 5;
  const int R = a.qg * a.T;
  const int n_occ = a.n_occ, n_keys = n_occ + a.T;
  const int kblocks = (n_keys + BK_KEYS - 1) / BK_KEYS;
  const int wi = xcd_remap(blockIdx.x, gridDim.x);
  const int grp = wi / kblocks, kbk = wi % kblocks;
  const int g = grp % a.Hkv, b = grp / a.Hkv;
  const int j_wg = kbk * BK_KEYS;
  const int j_base = j_wg + wave * 32;
  const int my_key = j_base + n;
  const bool key_ok = my_key < n_keys;
  const int t_key = my_key - n_occ;  // chunk position of the lane's key, < 0 for a cache slot
  // wave-uniform: all 32 keys of the wave exist; the chunk position of its last key
  const bool wave_keys_ok = j_base + 31 < n_keys;
  const int wave_tmax = j_base + 31 - n_occ;
  const size_t cache_row0 = static_cast<size_t>(grp) * a.C;
  const size_t new_row0 = static_cast<size_t>(grp) * a.T;
  const float sl2 = a.sl2;

  // K and V rows of the lane's key: B operands of S = Q K^T and dP = dO V^T
  bf16x8 kf[8], vf[8];
  {
    const int kk = key_ok ? my_key : 0;
    const size_t off = kk < n_occ ? (cache_row0 + kk) * ROW_BYTES : (new_row0 + (kk - n_occ)) * ROW_BYTES;
    const char *ks = static_cast<const char *>(kk < n_occ ? a.kc : a.kn) + off;
    const char *vs = static_cast<const char *>(kk < n_occ ? a.vc : a.vn) + off;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      kf[st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(ks + 32 * st + 16 * hl));
      vf[st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(vs + 32 * st + 16 * hl));
    }
  }

  // The group's rows r = i * q_g + hh live at (hh * T + i) rows from the
  // group's first query head (heads of a group are adjacent).
  const size_t head0 = static_cast<size_t>(b) * a.Hq + static_cast<size_t>(g) * a.qg;
  const rsrc_t q_rs = make_rsrc(static_cast<const char *>(a.q) + head0 * a.T * ROW_BYTES, R * ROW_BYTES);
  const rsrc_t g_rs = make_rsrc(static_cast<const char *>(a.dout) + head0 * a.T * ROW_BYTES, R * ROW_BYTES);
  const rsrc_t l_rs = make_rsrc(a.l2 + head0 * a.T, R * 4);
  const rsrc_t d_rs = make_rsrc(a.dd + head0 * a.T, R * 4);
  auto src_row = [&](int r) {  // offset in rows of packed row r (clamped to the last row)
    const int rr = r < R ? r : R - 1;
    return (rr % a.qg) * a.T + rr / a.qg;
  };
  auto issue_rows = [&](int rb, char *qdst, char *gdst, float *ldst, float *ddst) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int seg = wave * 4 + q;
      const int rib = seg * 4 + (lane >> 4);
      const uint32_t voff =
          static_cast<uint32_t>(src_row(rb + rib) * ROW_BYTES + 16 * bt_chunk_at(rib, lane & 15));
      dma16(q_rs, voff, 0, qdst + seg * 1024);
      dma16(g_rs, voff, 0, gdst + seg * 1024);
    }
    if (wave == 0) {
      const uint32_t off = static_cast<uint32_t>(src_row(rb + lane) * 4);
      dma4(l_rs, off, 0, reinterpret_cast<char *>(ldst));
      dma4(d_rs, off, 0, reinterpret_cast<char *>(ddst));
    }
  };

  const int r_first = j_wg >= n_occ ? (j_wg - n_occ) * a.qg : 0;  // first row any key of the block sees
  const int rb_begin = r_first / BR_ROWS * BR_ROWS;
  const int nrb = (R - rb_begin + BR_ROWS - 1) / BR_ROWS;
  const int prow = perm_key(n);

  f32x16 dv[4], dk[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    dv[k] = f32x16{};
    dk[k] = f32x16{};
  }

  auto compute = [&](int rb, const char *qb, const char *gb, const float *lb, const float *db) {
#pragma unroll 1
    for (int sub = 0; sub < 2; ++sub) {
      const char *qs = qb + sub * 32 * ROW_BYTES;
      const char *gs = gb + sub * 32 * ROW_BYTES;
      f32x16 c = f32x16{}, dp = f32x16{};
      bf16x8 qa = lds16(qs + bt_off(prow, hl)), ga = lds16(gs + bt_off(prow, hl));
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        bf16x8 nqa = qa, nga = ga;
        if (st < 7) {
          nqa = lds16(qs + bt_off(prow, 2 * st + 2 + hl));
          nga = lds16(gs + bt_off(prow, 2 * st + 2 + hl));
        }
        __builtin_amdgcn_sched_barrier(0);
        c = mfma32(qa, kf[st], c);
        dp = mfma32(ga, vf[st], dp);
        qa = nqa;
        ga = nga;
        __builtin_amdgcn_sched_barrier(0);
      }
      // register r: row rb + 32*sub + 16*(r/8) + 8*hl + r%8 of the lane's key
      const int r0 = rb + 32 * sub;
      const bool sub_full = wave_keys_ok && r0 + 31 < R && r0 >= wave_tmax * a.qg;
      bf16x8 pa[2], sa[2];
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        const int rib0 = 32 * sub + 16 * h8 + 8 * hl;
        const float4 L0 = *reinterpret_cast<const float4 *>(lb + rib0);
        const float4 L1 = *reinterpret_cast<const float4 *>(lb + rib0 + 4);
        const float4 D0 = *reinterpret_cast<const float4 *>(db + rib0);
        const float4 D1 = *reinterpret_cast<const float4 *>(db + rib0 + 4);
        const float Lv[8] = {L0.x, L0.y, L0.z, L0.w, L1.x, L1.y, L1.z, L1.w};
        const float Dv[8] = {D0.x, D0.y, D0.z, D0.w, D1.x, D1.y, D1.z, D1.w};
        if (sub_full) {  // every row of the sub-block sees all the wave's keys
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int r = 8 * h8 + e;
            const float p = __builtin_amdgcn_exp2f(fmaf(c[r], sl2, -Lv[e]));
            pa[h8][e] = static_cast<__bf16>(p);
            sa[h8][e] = static_cast<__bf16>(p * (dp[r] - Dv[e]));
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int r = 8 * h8 + e;
            const int row = rb + rib0 + e;
            const bool vis = key_ok && row < R && row >= t_key * a.qg;  // t_key < 0: every row
            const float p = vis ? __builtin_amdgcn_exp2f(fmaf(c[r], sl2, -Lv[e])) : 0.f;
            pa[h8][e] = static_cast<__bf16>(p);
            sa[h8][e] = static_cast<__bf16>(p * (dp[r] - Dv[e]));
          }
        }
      }
      // dV += P^T dO, dK += dS^T Q; k-step ks covers rows 16*ks .. 16*ks + 15 of the sub-block
      bf16x8 go = tr_operand(gs, 0, 0, lane), qo = tr_operand(qs, 0, 0, lane);
#pragma unroll
      for (int step = 0; step < 8; ++step) {
        const int ks = step >> 2, blk = step & 3;
        bf16x8 ngo = go, nqo = qo;
        if (step < 7) {
          ngo = tr_operand(gs, (step + 1) >> 2, (step + 1) & 3, lane);
          nqo = tr_operand(qs, (step + 1) >> 2, (step + 1) & 3, lane);
        }
        __builtin_amdgcn_sched_barrier(0);
        dv[blk] = mfma32(pa[ks], go, dv[blk]);
        dk[blk] = mfma32(sa[ks], qo, dk[blk]);
        go = ngo;
        qo = nqo;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  issue_rows(rb_begin, qb0, gb0, lb0, db0);
  for (int it = 0; it < nrb; it += 2) {
    const int rb = rb_begin + it * BR_ROWS;
    wait_dma_and_sync();  // block it in the 0 buffers; everybody done with the 1 buffers
    if (it + 1 < nrb) issue_rows(rb + BR_ROWS, qb1, gb1, lb1, db1);
    compute(rb, qb0, gb0, lb0, db0);
    if (it + 1 >= nrb) break;
    wait_dma_and_sync();
    if (it + 2 < nrb) issue_rows(rb + 2 * BR_ROWS, qb0, gb0, lb0, db0);
    compute(rb + BR_ROWS, qb1, gb1, lb1, db1);
  }

  // output register r of block blk: key j_base + 8*(r/4) + 4*hl + r%4, d = 32*blk + n
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int kk = j_base + 8 * (r >> 2) + 4 * hl + (r & 3);
    if (kk >= n_keys) continue;
    float *dkrow, *dvrow;
    if (kk < n_occ) {
      dkrow = a.dkc + (cache_row0 + kk) * D;
      dvrow = a.dvc + (cache_row0 + kk) * D;
    } else {
      dkrow = a.dkn + (new_row0 + (kk - n_occ)) * D;
      dvrow = a.dvn + (new_row0 + (kk - n_occ)) * D;
    }
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      dkrow[32 * blk + n] = dk[blk][r] * a.scale;
      dvrow[32 * blk + n] = dv[blk][r];
    }
  }
}

}  // namespace

hipError_t launch_attn_backward(const BwdArgs &a, hipStream_t s) {
  const int groups = a.B * a.Hkv;
  {
    const hipError_t e = launch_bwd_dq(a, s);
    if (e != hipSuccess) return e;
  }
  {
    KernelTimer timer(H2O_K_BWD_DKDV, s);
    const int n_keys = a.n_occ + a.T;
    hipLaunchKernelGGL(bwd_dkdv, dim3(groups * ((n_keys + BK_KEYS - 1) / BK_KEYS)), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace h2o
