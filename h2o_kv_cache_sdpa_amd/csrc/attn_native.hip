// bf16 attention passes for a native bf16 cache with head dimension 128 --
// the shape of the 16K/32K-slot workloads -- software-pipelined for gfx950.
//
// Same mathematics as attn_mfma.hip ("Learning how to Forget", §A.7: softmax
// of mask(d_h^{-1/2} Q K^T), output Y = m V, summed weights sum_i m_ij; §A.1
// mask with the chunk attending before it is written: cache slots visible,
// chunk keys causal), organised for throughput:
//
//  * K, V and Q tiles move HBM -> LDS with buffer_load_dwordx4 ... lds (no
//    staging registers).  Each lane's 16 bytes land at segment_base +
//    16*lane, so a tile's XOR swizzle is produced by choosing which global
//    chunk each lane fetches; the per-lane offset is a loop constant and the
//    tile position goes into the scalar offset.  The buffer form (rather than
//    global_load_lds) keeps the LDS-read counter in order, so a read issued
//    ahead of its use is waited for with lgkmcnt(N) instead of lgkmcnt(0).
//  * Operands read from LDS are fetched one MFMA step ahead of their use.
//  * V stays row-major [key][d] in LDS; the A operand of O^T = V^T P^T (keys
//    contiguous per lane) comes from ds_read_b64_tr_b16: within a 16-lane
//    group, lane k supplies V[kb + k/4][c0 + 4(k%4) .. +3] and lane i receives
//    V[kb + e][c0 + i], e = 0..3.
//  * Pass A keeps S for two tiles in flight: while the MFMAs of S(t+1) =
//    K(t+1) Q^T run, the VALU works on the softmax of S(t); then O^T +=
//    V(t)^T P(t)^T.  K tiles run one step ahead of V tiles in two LDS buffers
//    each; one barrier per tile.
//  * Pass B gives each wavefront 64 keys (two B-operand sets), so every Q
//    A-operand read from LDS feeds two MFMAs, and processes the exponentials
//    of one 32-row block while the next block's MFMAs run.
//
// LDS buffers are separate static arrays and every access names its buffer at
// compile time (loops are unrolled by the buffer parity), so the compiler can
// tell an in-flight DMA target from the buffer being read.

#include <algorithm>
#include <type_traits>

#include "device_util.hpp"
#include "h2o_internal.hpp"
#include "split_merge.hpp"
#include "tile_util.hpp"

namespace h2o {
namespace {

// Address of key row j of one KV group: cache slot j < n_occ, else chunk key
// j - n_occ (clamped to row 0 of the chunk beyond T; such keys are masked).
__device__ __forceinline__ const char *key_row(const void *cache, const void *chunk, size_t cache_row0,
                                               size_t new_row0, int n_occ, int T, int j) {
  if (j < n_occ) return static_cast<const char *>(cache) + (cache_row0 + j) * ROW_BYTES;
  const int t = j - n_occ;
  return static_cast<const char *>(chunk) + (new_row0 + (t < T ? t : 0)) * ROW_BYTES;
}

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int SG_VALU = 0x002, SG_MFMA = 0x008, SG_DS_READ = 0x100;

// ---------------------------------------------------------------------------
// Pass A: 128 packed query rows per block, 4 wavefronts x 32 rows
// ---------------------------------------------------------------------------

// NW: wavefronts per block (4 or 8), 32 rows each; a K/V tile serves them all.
template <int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void attn_a_native(AttnArgs a) {
  constexpr int ROWS = 32 * NW;  // packed rows per block
  constexpr int SPW = 16 / NW;   // 1 KB DMA segments of a 16 KB tile per wavefront
  __shared__ __attribute__((aligned(1024))) char kb0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char kb1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vb0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vb1[TILE_BYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, hl = lane >> 5;
  const int R = a.qg * a.T;
  const int tiles_per_grp = (R + ROWS - 1) / ROWS;
  const int wi_all = xcd_remap(blockIdx.x, gridDim.x);
  const int split = wi_all % a.nsplit;  // key split of this block (0 when unsplit)
  const int wi = wi_all / a.nsplit;
  // Row blocks go out last first: under the causal mask the last rows see the
  // most keys, and starting the longest blocks first evens out the tail.
  const int grp = wi / tiles_per_grp, rt = tiles_per_grp - 1 - wi % tiles_per_grp;
  const int g = grp % a.Hkv, b = grp / a.Hkv;
  const int row0 = rt * ROWS;
  const int wrow0 = row0 + wave * 32;
  const int my_row = wrow0 + n;
  const bool row_ok = my_row < R;
  const int i_q = row_ok ? my_row / a.qg : 0;
  const int h_q = g * a.qg + (row_ok ? my_row % a.qg : 0);
  const int n_occ = a.n_occ;
  const float sl2 = a.sl2;
  // wave-uniform: smallest chunk position of the wave's rows, and ragged rows
  const int wave_i_min = wrow0 / a.qg;
  const bool wave_ragged = wrow0 + 31 >= R;

  bf16x8 qf[8];
  {
    const uint16_t *qrow =
        static_cast<const uint16_t *>(a.q) + ((static_cast<size_t>(b) * a.Hq + h_q) * a.T + i_q) * D;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row_ok) v = *reinterpret_cast<const uint4 *>(qrow + 16 * st + 8 * hl);
      qf[st] = __builtin_bit_cast(bf16x8, v);
    }
  }

  const int last_row = min(R, row0 + ROWS) - 1;
  const int key_end = n_occ + last_row / a.qg + 1;
  // key tiles t_lo .. t_lo + ntiles - 1 of the block's range (all of it when unsplit)
  const int ntiles_all = (key_end + 63) / 64;
  int t_lo, ntiles;  // key tiles t_lo .. t_lo + ntiles - 1 of this split (ntiles 0: none)
  split_tiles(ntiles_all, a.nsplit, split, t_lo, ntiles);
  const size_t cache_row0 = static_cast<size_t>(grp) * a.C;
  const size_t new_row0 = static_cast<size_t>(grp) * a.T;

  // DMA of one 64-row tile: 16 segments of 1 KB (4 rows), 4 per wavefront.
  // Buffer resources span this group's n_occ cache rows and T chunk rows;
  // chunk rows past T read as zeros (and are masked).  A tile lying wholly in
  // the cache moves only the scalar offset.
  const rsrc_t kc_rs = make_rsrc(static_cast<const char *>(a.kc) + cache_row0 * ROW_BYTES, n_occ * ROW_BYTES);
  const rsrc_t vc_rs = make_rsrc(static_cast<const char *>(a.vc) + cache_row0 * ROW_BYTES, n_occ * ROW_BYTES);
  const rsrc_t kn_rs = make_rsrc(static_cast<const char *>(a.kn) + new_row0 * ROW_BYTES, a.T * ROW_BYTES);
  const rsrc_t vn_rs = make_rsrc(static_cast<const char *>(a.vn) + new_row0 * ROW_BYTES, a.T * ROW_BYTES);
  auto lane_off = [&](int q, bool is_v) -> uint32_t {
    const int row = (wave * SPW + q) * 4 + (lane >> 4);
    const int c = is_v ? v_chunk_at(row, lane & 15) : kq_chunk_at(row, lane & 15);
    return static_cast<uint32_t>(row * ROW_BYTES + 16 * c);
  };
  // Segments qa .. qb-1 of this wavefront's share of one tile.
  auto issue_segs = [&](int tile, char *dst, rsrc_t crs, rsrc_t nrs, bool is_v, int qa, int qb) {
    const int j0 = (t_lo + tile) * 64;
    if (j0 + 64 <= n_occ) {
#pragma unroll
      for (int q = qa; q < qb; ++q) dma16(crs, lane_off(q, is_v), j0 * ROW_BYTES, dst + (wave * SPW + q) * 1024);
    } else if (j0 >= n_occ) {  // chunk rows only
#pragma unroll
      for (int q = qa; q < qb; ++q)  // offset in voffset: rows past T fail the range check, read 0
        dma16(nrs, lane_off(q, is_v) + (j0 - n_occ) * ROW_BYTES, 0, dst + (wave * SPW + q) * 1024);
    } else {
      // the one tile that straddles n_occ: cache rows, then chunk rows
      const int dt = j0 - n_occ;  // chunk index of the tile's first row, < 0
#pragma unroll
      for (int q = qa; q < qb; ++q) {
        const int row = (wave * SPW + q) * 4 + (lane >> 4);
        const uint32_t lo = lane_off(q, is_v);
        if (dt + row >= 0) {
          dma16(nrs, lo + dt * ROW_BYTES, 0, dst + (wave * SPW + q) * 1024);
        } else {
          dma16(crs, lo + j0 * ROW_BYTES, 0, dst + (wave * SPW + q) * 1024);
        }
      }
    }
  };
  auto issue_k = [&](int tile, char *dst) { issue_segs(tile, dst, kc_rs, kn_rs, false, 0, SPW); };
  auto issue_v = [&](int tile, char *dst) { issue_segs(tile, dst, vc_rs, vn_rs, true, 0, SPW); };
  // Part p (0..3) of the loads issued during a tile: K segments for p < 2, V
  // segments for p >= 2, half of the wavefront's share each.  Spreading them
  // over the tile keeps 8 wavefronts from queueing 32 loads at one instant.
  auto issue_part = [&](int p, int tile_k, char *kdst, int tile_v, char *vdst) {
    constexpr int H = SPW / 2;
    if (p < 2) {
      if (tile_k >= 0) issue_segs(tile_k, kdst, kc_rs, kn_rs, false, p * H, (p + 1) * H);
    } else {
      if (tile_v >= 0) issue_segs(tile_v, vdst, vc_rs, vn_rs, true, (p - 2) * H, (p - 1) * H);
    }
  };

  const int prow = perm_key(n);
  const uint32_t k_lane = static_cast<uint32_t>(prow * ROW_BYTES + ((hl ^ (prow & 15)) << 4));
  const int grp16 = lane >> 4, i16 = lane & 15;
  f32x16 o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) o[k] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // S(0) alone (nothing to overlap with yet)
  auto s_only = [&](const char *kb, f32x16 &s0, f32x16 &s1) {
    s0 = f32x16{};
    s1 = f32x16{};
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const bf16x8 k0 = lds16(kb + kq_off(prow, 2 * st + hl));
      const bf16x8 k1 = lds16(kb + kq_off(32 + prow, 2 * st + hl));
      s0 = mfma32(k0, qf[st], s0);
      s1 = mfma32(k1, qf[st], s1);
    }
  };

  // Tile t: mask (diagonal tiles only), running max, lazy rescale; then, in
  // one straight-line block, the MFMAs of S(t+1) = K(t+1) Q^T from kb_next
  // interleaved with the exponentials of tile t, and O^T += V(t)^T P(t)^T.
  auto tile_step = [&](int t, f32x16 c0, f32x16 c1, const char *kb_next, f32x16 &n0, f32x16 &n1,
                       const char *vb, auto &&dma) {
    const int j0 = (t_lo + t) * 64;
    if (wave_ragged || j0 + 63 - n_occ > wave_i_min) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ja = j0 + 16 * (r >> 3) + 8 * hl + (r & 7) - n_occ;  // chunk index, < 0 for cache
        c0[r] = (row_ok && ja <= i_q) ? c0[r] : -INFINITY;
        c1[r] = (row_ok && ja + 32 <= i_q) ? c1[r] : -INFINITY;
      }
    }
    float mx = __builtin_fmaxf(__builtin_fmaxf(c0[0], c0[1]), c0[2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) mx = __builtin_fmaxf(__builtin_fmaxf(mx, c0[r]), c0[r + 1]);
    mx = __builtin_fmaxf(mx, c0[15]);
#pragma unroll
    for (int r = 0; r < 16; r += 2) mx = __builtin_fmaxf(__builtin_fmaxf(mx, c1[r]), c1[r + 1]);
    mx = max_xor32(mx * sl2);  // the other half-wave holds the row's other 32 keys
    if (__ballot(mx > m_run + RESCALE_SLACK)) {
      const float m_new = __builtin_fmaxf(m_run, mx);
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] *= alpha;
      m_run = m_new;
    }
    const float neg_m = (m_run == -INFINITY) ? 0.f : -m_run;

    // P(t) in four 16-key quarters: quarter ks holds keys 16ks .. 16ks+15 of
    // the lane's row, from S register c{ks/2}[8(ks&1) + e] (perm_key order).
    // Quarter ks's exponentials run beside S(t+1) steps 2ks, 2ks+1 and the
    // O^T += V^T P^T MFMAs of quarter ks-1, so that every stretch of the
    // tile has matrix and vector work in flight.
    bf16x8 pb[4];
    float ls[4] = {0.f, 0.f, 0.f, 0.f};
    n0 = f32x16{};
    n1 = f32x16{};
    // K operand of step st at k_lane ^ (st << 5) (rows prow and 32 + prow);
    // k_lane is made opaque per tile so that the eight addresses cost one
    // v_xor each instead of eight registers held across the loop.
    uint32_t ka = k_lane;
    asm volatile("" : "+v"(ka));
    // keys 16ks + 8h + 0..3 and + 4..7 at d = 32 blk + (lane % 32)
    auto v_operand = [&](int ks, int blk) {
      const int row = 16 * ks + 8 * (grp16 >> 1) + (i16 >> 2);
      const int col = 32 * blk + 16 * (grp16 & 1) + 4 * (i16 & 3);
      const bf16x4 lo = __builtin_bit_cast(bf16x4, lds_tr(vb + v_off(row, col >> 3) + 2 * (col & 7)));
      const bf16x4 hi = __builtin_bit_cast(bf16x4, lds_tr(vb + v_off(row + 4, col >> 3) + 2 * (col & 7)));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    bf16x8 kc0 = lds16(kb_next + ka), kc1 = lds16(kb_next + ka + 32 * ROW_BYTES);
    bf16x8 vc = kc0;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const f32x16 &cs = (ks < 2) ? c0 : c1;
      const int e0 = 8 * (ks & 1);
      dma(ks);
#pragma unroll
      for (int h = 0; h < 2; ++h) {  // S(t+1) step st = 2ks + h
        const int st = 2 * ks + h;
        bf16x8 kn0 = kc0, kn1 = kc1;
        if (st < 7) {
          const char *kp = kb_next + (ka ^ ((st + 1) << 5));
          kn0 = lds16(kp);
          kn1 = lds16(kp + 32 * ROW_BYTES);
        }
        if (ks > 0 && h == 0) vc = v_operand(ks - 1, 0);
        __builtin_amdgcn_sched_barrier(0);
        n0 = mfma32(kc0, qf[st], n0);
        n1 = mfma32(kc1, qf[st], n1);
        kc0 = kn0;
        kc1 = kn1;
#pragma unroll
        for (int e = 4 * h; e < 4 * h + 4; ++e) {
          const float p = __builtin_amdgcn_exp2f(fmaf(cs[e0 + e], sl2, neg_m));
          ls[ks] += p;
          pb[ks][e] = static_cast<__bf16>(p);
        }
        if (ks > 0) {  // O^T += V^T P^T for quarter ks-1, columns 64h .. 64h+63
#pragma unroll
          for (int b2 = 0; b2 < 2; ++b2) {
            const int blk = 2 * h + b2;
            const bf16x8 vn = (blk < 3) ? v_operand(ks - 1, blk + 1) : vc;
            o[blk] = mfma32(vc, pb[ks - 1], o[blk]);
            vc = vn;
          }
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(SG_VALU, 4, 0);
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(SG_VALU, 3, 0);
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(SG_VALU, 4, 0);
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(SG_VALU, 3, 0);
        } else {
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(SG_VALU, 7, 0);
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(SG_VALU, 7, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    // quarter 3: its MFMAs run on while the next tile's max is taken
    vc = v_operand(3, 0);
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      const bf16x8 vn = (blk < 3) ? v_operand(3, blk + 1) : vc;
      __builtin_amdgcn_sched_barrier(0);
      o[blk] = mfma32(vc, pb[3], o[blk]);
      vc = vn;
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- pipeline: K tiles one step ahead of V tiles, two LDS buffers each ----
  if (ntiles > 0) {
    issue_k(0, kb0);
    issue_v(0, vb0);
    if (ntiles > 1) issue_k(1, kb1);
    wait_dma_and_sync();
  }
  f32x16 sa0, sa1, sb0, sb1;  // S of the even / odd tile
  if (ntiles > 0) s_only(kb0, sa0, sa1);

  for (int t = 0; t < ntiles; t += 2) {
    // even tile t: K(t+1) in kb1, V(t) in vb0 (for the last tile, kb1 is stale
    // and the S it yields is discarded: one copy of the body per parity)
    wait_dma_and_sync();
    const int ke = t + 2 < ntiles ? t + 2 : -1, ve = t + 1 < ntiles ? t + 1 : -1;
    tile_step(t, sa0, sa1, kb1, sb0, sb1, vb0, [&](int p) { issue_part(p, ke, kb0, ve, vb1); });
    if (t + 1 >= ntiles) break;
    // odd tile t+1: K(t+2) in kb0, V(t+1) in vb1
    wait_dma_and_sync();
    const int ko = t + 3 < ntiles ? t + 3 : -1, vo = t + 2 < ntiles ? t + 2 : -1;
    tile_step(t + 1, sb0, sb1, kb0, sa0, sa1, vb1, [&](int p) { issue_part(p, ko, kb1, vo, vb0); });
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!row_ok) return;
  const size_t li = (static_cast<size_t>(b) * a.Hq + h_q) * a.T + i_q;
  if (a.nsplit > 1) {  // unnormalised partial output and (m, l) of this key split
    const size_t pr = static_cast<size_t>(split) * a.B * a.Hq * a.T + li;
    float *po = a.part + pr * D;
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d = 32 * blk + 8 * a4 + 4 * hl;
        *reinterpret_cast<float4 *>(po + d) =
            make_float4(o[blk][4 * a4], o[blk][4 * a4 + 1], o[blk][4 * a4 + 2], o[blk][4 * a4 + 3]);
      }
    }
    if (hl == 0) *reinterpret_cast<float2 *>(a.part_ml + 2 * pr) = make_float2(m_run, l_tot);
    return;
  }
  const float inv = 1.f / l_tot;
  H2O_DEVICE_CHECK(i_q < a.T && h_q < a.Hq && b < a.B);
  uint16_t *orow = static_cast<uint16_t *>(a.out) + li * D;
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int d = 32 * blk + 8 * a4 + 4 * hl;
      *reinterpret_cast<uint2 *>(orow + d) =
          make_uint2(pack_bf16_rne(o[blk][4 * a4] * inv, o[blk][4 * a4 + 1] * inv),
                     pack_bf16_rne(o[blk][4 * a4 + 2] * inv, o[blk][4 * a4 + 3] * inv));
    }
  }
  if (hl == 0) {
    const float L = m_run + log2f(l_tot);
    a.lse2[li] = L;
    if (a.lse_nat) a.lse_nat[li] = L * 0.69314718055994530942f;
  }
}

// Merge of the key splits of pass A: per row, M = max_s m_s,
// l = sum_s l_s 2^(m_s - M), out = sum_s 2^(m_s - M) O_s / l, L = M + log2 l
// (the same rescaling the online softmax applies between tiles).  A row is
// served by sg = min(nsplit, 8) groups of 32 lanes (4 components each); group
// k takes splits k, k + sg, ...; the groups' sums are added in group order, so
// the result does not depend on timing.  256 threads = 8 / sg rows.
__global__ __launch_bounds__(256) void attn_combine(AttnArgs a) {
  __shared__ float red_m[8], red_l[8];
  __shared__ float4 red_o[8][32];
  const size_t rows = static_cast<size_t>(a.B) * a.Hq * a.T;
  const int ns = a.nsplit;
  const int sg = ns < 8 ? ns : 8;
  const int slot = threadIdx.x >> 5, c = threadIdx.x & 31;
  const int rloc = slot / sg, sl = slot % sg;
  const size_t row = static_cast<size_t>(blockIdx.x) * (8 / sg) + rloc;
  const bool ok = rloc < 8 / sg && row < rows;
  // nsplit <= 64 = 8 lane groups x MAXI: every load of a lane group is issued
  // before the first one is used
  constexpr int MAXI = 8;
  float ms[MAXI], ls[MAXI];
  float4 po[MAXI];
#pragma unroll
  for (int i = 0; i < MAXI; ++i) {
    const int sp = sl + i * sg;
    ms[i] = -INFINITY;
    ls[i] = 0.f;
    po[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (ok && sp < ns) {
      const size_t pr = sp * rows + row;
      const float2 v = *reinterpret_cast<const float2 *>(a.part_ml + 2 * pr);
      ms[i] = v.x;
      ls[i] = v.y;
      po[i] = *reinterpret_cast<const float4 *>(a.part + pr * D + 4 * c);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < MAXI; ++i) M = fmaxf(M, ms[i]);
  if (c == 0) red_m[slot] = M;
  __syncthreads();
  if (ok)
    for (int k = 0; k < sg; ++k) M = fmaxf(M, red_m[rloc * sg + k]);
  float l = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int i = 0; i < MAXI; ++i) {
    if (ms[i] == -INFINITY) continue;  // no visible key in this split (or no split)
    const float wgt = __builtin_amdgcn_exp2f(ms[i] - M);
    l = fmaf(ls[i], wgt, l);
    acc.x = fmaf(po[i].x, wgt, acc.x);
    acc.y = fmaf(po[i].y, wgt, acc.y);
    acc.z = fmaf(po[i].z, wgt, acc.z);
    acc.w = fmaf(po[i].w, wgt, acc.w);
  }
  red_o[slot][c] = acc;
  if (c == 0) red_l[slot] = l;
  __syncthreads();
  if (!ok || sl != 0) return;
  for (int k = 1; k < sg; ++k) {
    const float4 o = red_o[slot + k][c];
    acc.x += o.x;
    acc.y += o.y;
    acc.z += o.z;
    acc.w += o.w;
    l += red_l[slot + k];
  }
  const float inv = 1.f / l;
  uint16_t *orow = static_cast<uint16_t *>(a.out) + row * D;
  *reinterpret_cast<uint2 *>(orow + 4 * c) =
      make_uint2(pack_bf16_rne(acc.x * inv, acc.y * inv), pack_bf16_rne(acc.z * inv, acc.w * inv));
  if (c == 0) {
    const float L = M + log2f(l);
    a.lse2[row] = L;
    if (a.lse_nat) a.lse_nat[row] = L * 0.69314718055994530942f;
  }
}

// ---------------------------------------------------------------------------
// Summed weights of short chunks from the logits pass A stored: one thread per
// key, rows of the KV group in order, Kahan-compensated like pass B.  Key j is
// visible to row r (chunk position r / qg) when it is a cache slot or a chunk
// key at a position <= r / qg.
// ---------------------------------------------------------------------------
// xs: factor that brings a stored logit to log2 units (sl2 for native caches,
// whose pass A stores q.k; 1 for 8/4-bit caches, whose factors include sl2).
// With key-split partials (nsplit > 1) the kernel also does the split
// combine: every block forms its group's row normalisers from the partial
// (m, l) pairs, and block x < R of a group merges output row x (the
// attn_combine arithmetic for that row), so no separate combine runs.
__global__ __launch_bounds__(256) void attn_b_logits(AttnArgs a, float xs) {
  __shared__ float Ls[LOGIT_ROWS_MAX], Ms[LOGIT_ROWS_MAX], Ws[LOGIT_ROWS_MAX];
  __shared__ float4 red_o[8][32];
  const int grp = blockIdx.y, g = grp % a.Hkv, b = grp / a.Hkv;
  const int R = a.qg * a.T;
  const int tid = threadIdx.x;
  const size_t rows = static_cast<size_t>(a.B) * a.Hq * a.T;
  auto row_index = [&](int r) {
    return (static_cast<size_t>(b) * a.Hq + g * a.qg + r % a.qg) * a.T + r / a.qg;
  };
  if (a.nsplit > 1) {  // 16 lanes per row, all loads issued before use
    const int r = tid >> 4, sl = tid & 15;
    float2 ml[4];
    load_split_ml(a, rows, r < R ? row_index(r) : 0, sl, r < R, ml);
    float M, W;
    reduce_split_ml(ml, M, W);
    if (r < R && sl == 0) {
      Ms[r] = M;
      Ws[r] = W;
      Ls[r] = M + log2f(W);
    }
  } else if (tid < R) {
    Ls[tid] = a.lse2[row_index(tid)];
  }
  __syncthreads();
  if (a.nsplit > 1 && static_cast<int>(blockIdx.x) < R) {  // output row x
    const int r = blockIdx.x, q = tid >> 5, c4 = tid & 31;
    const size_t li = row_index(r);
    float ms[8];
    float4 po[8];
    load_split_row(a, rows, li, q, c4, true, ms, po);
    merge_split_row(a, li, Ms[r], Ws[r], Ls[r], q, c4, true, ms, po, red_o);
  }
  const int n_keys = a.n_occ + a.T;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= n_keys) return;
  const float *src = a.lg + static_cast<size_t>(grp) * R * a.lg_stride + j;
  const int t = j - a.n_occ;  // chunk position of the key, < 0 for cache slots
  float x[LOGIT_ROWS_MAX];
#pragma unroll
  for (int r = 0; r < LOGIT_ROWS_MAX; ++r) x[r] = r < R ? src[static_cast<size_t>(r) * a.lg_stride] : 0.f;
  a.wsum[static_cast<size_t>(grp) * n_keys + j] = key_weight_sum(
      R, [&](int r) { return x[r]; }, [&](int r) { return t * a.qg <= r - r % a.qg; }, xs, Ls);  // t <= r / qg
}

// ---------------------------------------------------------------------------
// Pass B: 256 keys per block, 4 wavefronts x 64 keys; 128-row Q blocks
// ---------------------------------------------------------------------------

constexpr int PB_KEYS = 256;
constexpr int PB_ROWS = 128;
constexpr int SLICE_KEYS = 32;  // chunk keys folded into one key block
constexpr int PB_PLAIN = 0, PB_FOLD = 1, PB_PAIR = 2;  // attn_b_native work mappings
constexpr int QBLK_BYTES = PB_ROWS * ROW_BYTES;  // 32 KB

// 8 codes of one key row (int8: 8 bytes, int4: 4 bytes with element 2k in the
// low nibble of byte k) -> 8 bf16; integers are exact in bf16.
template <int FMT>
__device__ __forceinline__ bf16x8 widen8(const char *codes) {
  uint32_t r[4];
  if constexpr (FMT == FMT_INT8) {
    const uint2 c = *reinterpret_cast<const uint2 *>(codes);
    const uint32_t w[2] = {c.x, c.y};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int32_t x = static_cast<int32_t>(w[h]);
      const float f0 = static_cast<float>((x << 24) >> 24), f1 = static_cast<float>((x << 16) >> 24);
      const float f2 = static_cast<float>((x << 8) >> 24), f3 = static_cast<float>(x >> 24);
      r[2 * h] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
      r[2 * h + 1] = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
    }
  } else {
    const uint32_t w = *reinterpret_cast<const uint32_t *>(codes);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t byte = (w >> (8 * q)) & 0xffu;
      const float lo = static_cast<float>(byte & 15u), hi = static_cast<float>(byte >> 4);
      r[q] = __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
    }
  }
  return __builtin_bit_cast(bf16x8, make_uint4(r[0], r[1], r[2], r[3]));
}

// FMT: cache format.  For 8/4-bit caches the K operands are the widened codes
// and the per-key factors enter the exponent: x = s_j*sl2*acc (+ z_j*sl2*sum(q_i)) - L_i.
//
// SL (folded chunk keys): blocks are launched only for the key blocks that
// start below n_occ, which see every query row.  The keys past them (chunk
// keys only, visible to a shrinking suffix of the rows) would otherwise form a
// few extra blocks that run as a nearly empty last wave of the grid; instead
// they are cut into 32-key slices and block k also sums slice k: wavefront w
// takes 32-row sub-block w of every row block against the slice's keys, which
// sit in LDS for the whole block, and the four partial column sums are added
// in a fixed order at the end.
template <int FMT, int MODE>
__global__ __launch_bounds__(256, 2) void attn_b_native(AttnArgs a) {
  constexpr bool SL = MODE == PB_FOLD, PAIR = MODE == PB_PAIR;
  __shared__ __attribute__((aligned(1024))) char qb0[QBLK_BYTES];
  __shared__ __attribute__((aligned(1024))) char qb1[QBLK_BYTES];
  __shared__ __attribute__((aligned(1024))) char sk[SL ? SLICE_KEYS * ROW_BYTES : 16];
  __shared__ float sred[SL ? 4 * SLICE_KEYS : 1];
  __shared__ __attribute__((aligned(512))) float lb0[PB_ROWS];
  __shared__ __attribute__((aligned(512))) float lb1[PB_ROWS];
  // int4: per-row sum(q) beside the normalisers
  __shared__ __attribute__((aligned(512))) float sb0[FMT == FMT_INT4 ? PB_ROWS : 1];
  __shared__ __attribute__((aligned(512))) float sb1[FMT == FMT_INT4 ? PB_ROWS : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, hl = lane >> 5;
  const int n_occ = a.n_occ;
  const int n_keys = n_occ + a.T;
  const int R = a.qg * a.T;
  const int n_main = (n_occ + PB_KEYS - 1) / PB_KEYS;  // key blocks starting below n_occ
  const int kblocks_all = (n_keys + PB_KEYS - 1) / PB_KEYS;
  const int kblocks = SL ? n_main : PAIR ? (kblocks_all + 1) / 2 : kblocks_all;  // work items per group
  const int wi = xcd_remap(blockIdx.x, gridDim.x);
  const int grp = wi / kblocks, item = wi % kblocks;
  const int g = grp % a.Hkv, b = grp / a.Hkv;
  // PAIR: item i sums key blocks i and kblocks_all - 1 - i, one after the other
  const int npass = (PAIR && item != kblocks_all - 1 - item) ? 2 : 1;
#pragma unroll 1
  for (int pass = 0; pass < npass; ++pass) {
    const int kbk = pass == 0 ? item : kblocks_all - 1 - item;
    if (pass > 0) __syncthreads();  // every wavefront is done with the LDS row buffers
    const int j_base = kbk * PB_KEYS;
    const size_t cache_row0 = static_cast<size_t>(grp) * a.C;
    const size_t new_row0 = static_cast<size_t>(grp) * a.T;
    const float sl2 = a.sl2;

    // K^T operands of the wave's two 32-key sub-blocks
    int key0 = j_base + wave * 64 + n, key1 = key0 + 32;
    const int tnew0 = key0 - n_occ, tnew1 = key1 - n_occ;
    bf16x8 kf0[8], kf1[8];
    // per-key factors of the exponent: sl2 * s_k, sl2 * z_k (chunk keys: sl2, 0)
    float ksl0 = sl2, ksl1 = sl2, kzl0 = 0.f, kzl1 = 0.f;
    if constexpr (FMT == FMT_NATIVE) {
      const char *src0 = key_row(a.kc, a.kn, cache_row0, new_row0, n_occ, a.T, key0 < n_keys ? key0 : 0);
      const char *src1 = key_row(a.kc, a.kn, cache_row0, new_row0, n_occ, a.T, key1 < n_keys ? key1 : 0);
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        kf0[st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(src0 + 32 * st + 16 * hl));
        kf1[st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(src1 + 32 * st + 16 * hl));
      }
    } else {
      constexpr int CROW = (FMT == FMT_INT8) ? D : D / 2;  // code bytes per key
      auto load_key = [&](int key, bf16x8 (&kf)[8], float &ksl, float &kzl) {
        const int kk = key < n_keys ? key : 0;
        if (kk < n_occ) {
          const char *src = static_cast<const char *>(a.kc) + (cache_row0 + kk) * CROW;
#pragma unroll
          for (int st = 0; st < 8; ++st) kf[st] = widen8<FMT>(src + (16 * st + 8 * hl) * CROW / D);
          ksl = f16_to_f32(a.ks[cache_row0 + kk]) * sl2;
          if constexpr (FMT == FMT_INT4) kzl = f16_to_f32(a.kz[cache_row0 + kk]) * sl2;
        } else {
          const char *src = key_row(a.kc, a.kn, cache_row0, new_row0, n_occ, a.T, kk);
#pragma unroll
          for (int st = 0; st < 8; ++st)
            kf[st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(src + 32 * st + 16 * hl));
        }
      };
      load_key(key0, kf0, ksl0, kzl0);
      load_key(key1, kf1, ksl1, kzl1);
    }

    // Slice kbk: keys s_key0 .. s_key0 + 31 (those below n_keys), chunk
    // positions ts0 + n; row r sees key n of the slice iff r >= (ts0 + n) * q_g.
    const int s_key0 = n_main * PB_KEYS + SLICE_KEYS * kbk;
    const int ts0 = s_key0 - n_occ;
    const bool has_slice = SL && s_key0 < n_keys;
    const int s_first = (ts0 + n) * a.qg;
    if (has_slice) {  // 8 segments of 4 rows, same chunk swizzle as a Q block
      const rsrc_t kn_rs = make_rsrc(static_cast<const char *>(a.kn) + new_row0 * ROW_BYTES, a.T * ROW_BYTES);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int seg = wave * 2 + q;
        const int rr = seg * 4 + (lane >> 4);
        const int t = ts0 + rr < a.T ? ts0 + rr : a.T - 1;  // keys past the chunk: any row, never written
        dma16(kn_rs, t * ROW_BYTES + 16 * kq_chunk_at(rr, lane & 15), 0, sk + seg * 1024);
      }
    }
    float sacc = 0.f, scomp = 0.f;

    const int row_first = (j_base >= n_occ) ? (j_base - n_occ) * a.qg : 0;
    const int rb_begin = row_first / PB_ROWS * PB_ROWS;
    const int nrb = (R - rb_begin + PB_ROWS - 1) / PB_ROWS;
    const int t_last = j_base + PB_KEYS - 1 - n_occ;
    const size_t lse_base = static_cast<size_t>(b) * a.Hq * a.T;

    // DMA of a 128-row Q block (32 KB: 32 segments, 8 per wavefront) and its
    // normalisers.  When q_g divides the block height, row rb + rr is query
    // rb/q_g + rr/q_g of head g*q_g + rr%q_g: a per-lane constant offset plus a
    // wave-uniform base.
    const bool rows_split = (PB_ROWS % a.qg) == 0;
    // The group's q_g query heads (q_g*T rows of Q) and their normalisers are
    // contiguous: row r = i*q_g + hh lives at (hh*T + i).
    const rsrc_t q_rs = make_rsrc(static_cast<const char *>(a.q) +
                                      (static_cast<size_t>(b) * a.Hq + static_cast<size_t>(g) * a.qg) * a.T * ROW_BYTES,
                                  R * ROW_BYTES);
    const rsrc_t l_rs = make_rsrc(a.lse2 + lse_base + static_cast<size_t>(g) * a.qg * a.T, R * 4);
    const rsrc_t s_rs = make_rsrc(a.lse2 + static_cast<size_t>(a.B) * a.Hq * a.T + lse_base +
                                      static_cast<size_t>(g) * a.qg * a.T,
                                  R * 4);
    uint32_t qoff[8];
    uint32_t loff = 0;
    if (rows_split) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int rr = (wave * 8 + q) * 4 + (lane >> 4);
        qoff[q] = ((rr % a.qg) * a.T + rr / a.qg) * ROW_BYTES + 16 * kq_chunk_at(rr, lane & 15);
      }
      const int rl = (wave & 1) * 64 + lane;
      loff = ((rl % a.qg) * a.T + rl / a.qg) * 4;
    }
    // L rows by waves 0-1; for int4 the sum(q) rows by waves 2-3
    auto issue_rows = [&](int rb, char *qdst, float *ldst, float *sdst) {
      if (rows_split && rb + PB_ROWS <= R) {
        const uint32_t shift = static_cast<uint32_t>(rb / a.qg);
#pragma unroll
        for (int q = 0; q < 8; ++q) dma16(q_rs, qoff[q], shift * ROW_BYTES, qdst + (wave * 8 + q) * 1024);
        if (wave < 2) {
          dma4(l_rs, loff, shift * 4, reinterpret_cast<char *>(ldst + wave * 64));
        } else if (FMT == FMT_INT4) {
          dma4(s_rs, loff, shift * 4, reinterpret_cast<char *>(sdst + (wave - 2) * 64));
        }
        return;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int seg = wave * 8 + q;
        const int rr = seg * 4 + (lane >> 4);
        int row = rb + rr;
        row = row < R ? row : R - 1;  // rows past the end are masked
        const int ii = row / a.qg, hh = row % a.qg;
        dma16(q_rs, (hh * a.T + ii) * ROW_BYTES + 16 * kq_chunk_at(rr, lane & 15), 0, qdst + seg * 1024);
      }
      {
        int row = rb + (wave & 1) * 64 + lane;
        row = row < R ? row : R - 1;
        const int ii = row / a.qg, hh = row % a.qg;
        if (wave < 2) {
          dma4(l_rs, (hh * a.T + ii) * 4, 0, reinterpret_cast<char *>(ldst + wave * 64));
        } else if (FMT == FMT_INT4) {
          dma4(s_rs, (hh * a.T + ii) * 4, 0, reinterpret_cast<char *>(sdst + (wave - 2) * 64));
        }
      }
    };

    float acc0 = 0.f, comp0 = 0.f, acc1 = 0.f, comp1 = 0.f;
    auto add_comp = [](float &acc, float &comp, float part) {
      const float y = part - comp;
      const float tt = acc + y;
      comp = (tt - acc) - y;
      acc = tt;
    };
    auto load_l = [&](const float *lb, int sub, float (&Lv)[16]) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const float4 L = *reinterpret_cast<const float4 *>(lb + 32 * sub + 8 * a4 + 4 * hl);
        Lv[4 * a4] = L.x;
        Lv[4 * a4 + 1] = L.y;
        Lv[4 * a4 + 2] = L.z;
        Lv[4 * a4 + 3] = L.w;
      }
    };

    const uint32_t q_lane = static_cast<uint32_t>(n * ROW_BYTES + ((hl ^ (n & 15)) << 4));
    // Row r sees chunk key t iff floor(r / q_g) >= t, i.e. r >= t * q_g.
    const int first_row0 = tnew0 > 0 ? tnew0 * a.qg : 0;
    const int first_row1 = tnew1 > 0 ? tnew1 * a.qg : 0;

    // One 128-row block: the MFMAs of sub-block k+1 run while the VALU sums
    // the exponentials of sub-block k.  FULL: every row sees every key.
    auto do_block = [&](auto full_tag, const char *qb, const float *lb, const float *sb, int rb) {
      constexpr bool FULL = decltype(full_tag)::value;
      // Q operand of sub-block sub, step st: sub * 32 rows + (q_lane ^ (st << 5));
      // q_lane is made opaque per block (one v_xor per read, no held addresses).
      uint32_t qa_l = q_lane;
      asm volatile("" : "+v"(qa_l));
      auto qop = [&](int sub, int st) { return lds16(qb + sub * (32 * ROW_BYTES) + (qa_l ^ (st << 5))); };
      f32x16 c0 = f32x16{}, c1 = f32x16{};
      float Lc[16], Sc[16];
      bf16x8 qc = qop(0, 0);
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const bf16x8 qn = st < 7 ? qop(0, st + 1) : qop(1, 0);
        __builtin_amdgcn_sched_barrier(0);
        c0 = mfma32(qc, kf0[st], c0);
        c1 = mfma32(qc, kf1[st], c1);
        qc = qn;
        __builtin_amdgcn_sched_barrier(0);
      }
      load_l(lb, 0, Lc);
      if constexpr (FMT == FMT_INT4) load_l(sb, 0, Sc);
#pragma unroll
      for (int sub = 1; sub <= 4; ++sub) {
        f32x16 n0 = f32x16{}, n1 = f32x16{};
        float p0[2] = {0.f, 0.f}, p1[2] = {0.f, 0.f};
        const int rsub = rb + 32 * (sub - 1);  // rows of the block being summed
#pragma unroll
        for (int st = 0; st < 8; ++st) {
          if (sub < 4) {
            bf16x8 qn = qc;
            if (st < 7) {
              qn = qop(sub, st + 1);
            } else if (sub < 3) {
              qn = qop(sub + 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            n0 = mfma32(qc, kf0[st], n0);
            n1 = mfma32(qc, kf1[st], n1);
            qc = qn;
          }
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int r = 2 * st + h2;
            float x0, x1;
            if constexpr (FMT == FMT_NATIVE) {
              x0 = fmaf(c0[r], sl2, -Lc[r]);
              x1 = fmaf(c1[r], sl2, -Lc[r]);
            } else if constexpr (FMT == FMT_INT8) {
              x0 = fmaf(c0[r], ksl0, -Lc[r]);
              x1 = fmaf(c1[r], ksl1, -Lc[r]);
            } else {
              x0 = fmaf(c0[r], ksl0, fmaf(kzl0, Sc[r], -Lc[r]));
              x1 = fmaf(c1[r], ksl1, fmaf(kzl1, Sc[r], -Lc[r]));
            }
            if constexpr (!FULL) {
              const int row = rsub + 8 * (r >> 2) + 4 * hl + (r & 3);
              x0 = (row < R && row >= first_row0) ? x0 : -INFINITY;
              x1 = (row < R && row >= first_row1) ? x1 : -INFINITY;
            }
            p0[h2] += __builtin_amdgcn_exp2f(x0);
            p1[h2] += __builtin_amdgcn_exp2f(x1);
          }
          if (sub < 4) {
            __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
            __builtin_amdgcn_sched_group_barrier(SG_VALU, FULL ? 6 : 10, 0);
            __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
            __builtin_amdgcn_sched_group_barrier(SG_VALU, FULL ? 6 : 10, 0);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        add_comp(acc0, comp0, p0[0] + p0[1]);
        add_comp(acc1, comp1, p1[0] + p1[1]);
        if (sub < 4) {
          c0 = n0;
          c1 = n1;
          load_l(lb, sub, Lc);
          if constexpr (FMT == FMT_INT4) load_l(sb, sub, Sc);
        }
      }
    };
    // The slice against this wavefront's 32 rows of the block.  The slice keys
    // are chunk keys in bf16, so x = acc * sl2 - L for every cache format.
    auto slice_rows = [&](const char *qb, const float *lb, int rb) {
      const int r0 = rb + 32 * wave;
      if (r0 >= R || r0 + 31 < ts0 * a.qg) return;  // no row here sees a slice key
      uint32_t qa_l = q_lane;
      asm volatile("" : "+v"(qa_l));
      const char *qs = qb + wave * (32 * ROW_BYTES);
      f32x16 cs = f32x16{};
      bf16x8 qa = lds16(qs + qa_l), ka = lds16(sk + qa_l);
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        bf16x8 qn = qa, kn = ka;
        if (st < 7) {
          qn = lds16(qs + (qa_l ^ ((st + 1) << 5)));
          kn = lds16(sk + (qa_l ^ ((st + 1) << 5)));
        }
        cs = mfma32(qa, ka, cs);
        qa = qn;
        ka = kn;
      }
      float Ls[16];
      load_l(lb, wave, Ls);
      const bool sfull = r0 + 31 < R && r0 >= (ts0 + SLICE_KEYS - 1) * a.qg;
      float ps[2] = {0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = fmaf(cs[r], sl2, -Ls[r]);
        if (!sfull) {
          const int row = r0 + 8 * (r >> 2) + 4 * hl + (r & 3);
          x = (row < R && row >= s_first) ? x : -INFINITY;
        }
        ps[r & 1] += __builtin_amdgcn_exp2f(x);
      }
      add_comp(sacc, scomp, ps[0] + ps[1]);
    };
    auto block = [&](const char *qb, const float *lb, const float *sb, int rb) {
      const bool full = (rb + PB_ROWS <= R) && (j_base + PB_KEYS <= n_occ || rb / a.qg >= t_last);
      if (full) {
        do_block(std::true_type{}, qb, lb, sb, rb);
      } else {
        do_block(std::false_type{}, qb, lb, sb, rb);
      }
      if constexpr (SL) {
        if (has_slice) slice_rows(qb, lb, rb);
      }
    };

    issue_rows(rb_begin, qb0, lb0, sb0);
    for (int it = 0; it < nrb; it += 2) {
      const int rb = rb_begin + it * PB_ROWS;
      wait_dma_and_sync();  // block it in qb0; everybody done with qb1
      if (it + 1 < nrb) issue_rows(rb + PB_ROWS, qb1, lb1, sb1);
      block(qb0, lb0, sb0, rb);
      if (it + 1 >= nrb) break;
      wait_dma_and_sync();  // block it+1 in qb1; everybody done with qb0
      if (it + 2 < nrb) issue_rows(rb + 2 * PB_ROWS, qb0, lb0, sb0);
      block(qb1, lb1, sb1, rb + PB_ROWS);
    }

    const float mine0 = acc0 - comp0, mine1 = acc1 - comp1;
    const float other0 = __shfl_xor(mine0, 32), other1 = __shfl_xor(mine1, 32);
    if (hl == 0) {
      float *w = a.wsum + static_cast<size_t>(grp) * n_keys;
      H2O_DEVICE_CHECK(grp < a.B * a.Hkv && key0 >= 0 && key1 >= 0);
      if (key0 < n_keys) w[key0] = mine0 + other0;
      if (key1 < n_keys) w[key1] = mine1 + other1;
    }
    if constexpr (SL) {
      if (has_slice) {
        const float sm = sacc - scomp;
        const float so = __shfl_xor(sm, 32);
        if (hl == 0) sred[wave * SLICE_KEYS + n] = sm + so;
        __syncthreads();
        if (wave == 0 && hl == 0 && s_key0 + n < n_keys) {
          const float tot = ((sred[n] + sred[SLICE_KEYS + n]) + sred[2 * SLICE_KEYS + n]) + sred[3 * SLICE_KEYS + n];
          a.wsum[static_cast<size_t>(grp) * n_keys + s_key0 + n] = tot;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_attn_combine(const AttnArgs &a, hipStream_t s) {
  const size_t rows = static_cast<size_t>(a.B) * a.Hq * a.T;
  const int rpb = 8 / (a.nsplit < 8 ? a.nsplit : 8);  // rows per block
  KernelTimer timer(H2O_K_ATTN_COMBINE, s);
  hipLaunchKernelGGL(attn_combine, dim3(static_cast<unsigned>((rows + rpb - 1) / rpb)), dim3(256), 0, s, a);
  return hipGetLastError();
}

int attn_splits(int B, int Hq, int Hkv, int D, int T, int n_occ, int dtype, int cache_fmt) {
  (void)cache_fmt;
  if (dtype != DT_BF16 || D != 128) return 1;
  // 2 blocks of pass A per CU on 256 CUs; split the keys of each row block
  // until the grid fills them, keeping at least 4 key tiles per split.
  constexpr int kSlots = 512;
  const long long blocks = static_cast<long long>(B) * Hkv * (((Hq / Hkv) * T + 127) / 128);
  const int tiles = (n_occ + T + 63) / 64;
  int ns = static_cast<int>((kSlots + blocks - 1) / blocks);
  ns = std::min(ns, std::max(1, tiles / 4));
  return std::max(1, std::min(ns, 64));
}

size_t attn_split_floats(int B, int Hq, int D, int T, int nsplit) {
  if (nsplit <= 1) return 0;
  return static_cast<size_t>(nsplit) * B * Hq * T * (D + 2);
}

hipError_t launch_attn_native_d128(const AttnArgs &a, hipStream_t s) {
  const int groups = a.B * a.Hkv;
  const int R = a.qg * a.T;
  const int nA = groups * ((R + 127) / 128) * a.nsplit;
  hipError_t e;
  {
    KernelTimer timer(H2O_K_ATTN_A, s);
    if (R <= 16) {  // short chunks: 16 keys of each tile per wavefront (attn_short.hip)
      e = launch_attn_a_short_d128(a, s);
    } else {
      if (R >= 256) {  // long chunks: 256 rows per block share each tile
        const int n8 = groups * ((R + 255) / 256) * a.nsplit;
        hipLaunchKernelGGL((attn_a_native<8>), dim3(n8), dim3(512), 0, s, a);
      } else {
        hipLaunchKernelGGL((attn_a_native<4>), dim3(nA), dim3(256), 0, s, a);
      }
      e = hipGetLastError();
    }
  }
  if (e != hipSuccess) return e;
  // with stored logits the weight-sum kernel also merges the key splits
  if (a.nsplit > 1 && !a.lg) {
    e = launch_attn_combine(a, s);
    if (e != hipSuccess) return e;
  }
  if (!a.wsum || (a.lg && a.defer_b)) return hipSuccess;
  if (a.lg) return launch_attn_b_logits(a, s);
  return launch_attn_b_native(a, s);
}

hipError_t launch_attn_b_logits(const AttnArgs &a, hipStream_t s) {
  const int n_keys = a.n_occ + a.T;
  // grid.x >= R, so that the blocks merging the split rows exist
  const int nx = std::max((n_keys + 255) / 256, a.qg * a.T);
  KernelTimer timer(H2O_K_ATTN_B, s);
  const float xs = a.cache_fmt == FMT_NATIVE ? a.sl2 : 1.f;
  hipLaunchKernelGGL(attn_b_logits, dim3(nx, a.B * a.Hkv), dim3(256), 0, s, a, xs);
  return hipGetLastError();
}

// Fold the chunk-only keys into the full key blocks when there is a full
// block for every 32-key slice and folding lowers the number of blocks the
// busiest of the 256 CUs runs (a CU's throughput is about the same with one
// or two resident blocks, so that count sets the kernel's duration).
static bool fold_chunk_keys(const AttnArgs &a) {
  constexpr long long kCUs = 256;
  const int n_keys = a.n_occ + a.T;
  const int n_main = (a.n_occ + PB_KEYS - 1) / PB_KEYS;
  const int slices = (n_keys - n_main * PB_KEYS + SLICE_KEYS - 1) / SLICE_KEYS;
  const long long groups = static_cast<long long>(a.B) * a.Hkv;
  const long long per_cu = (groups * ((n_keys + PB_KEYS - 1) / PB_KEYS) + kCUs - 1) / kCUs;
  const long long per_cu_fold = (groups * n_main + kCUs - 1) / kCUs;
  return a.n_occ > 0 && slices >= 1 && slices <= n_main && per_cu_fold < per_cu;
}

// An empty cache (a prefill chunk): key block k sees the rows from k*256/q_g
// on, a linear profile, so blocks k and K-1-k together make one even item.
template <int FMT>
static void launch_b_fmt(const AttnArgs &a, hipStream_t s) {
  const int groups = a.B * a.Hkv;
  const int kblocks = (a.n_occ + a.T + PB_KEYS - 1) / PB_KEYS;
  if (fold_chunk_keys(a)) {
    const int nB = groups * ((a.n_occ + PB_KEYS - 1) / PB_KEYS);
    hipLaunchKernelGGL((attn_b_native<FMT, PB_FOLD>), dim3(nB), dim3(256), 0, s, a);
  } else if (a.n_occ == 0 && kblocks >= 2) {
    const int nB = groups * ((kblocks + 1) / 2);
    hipLaunchKernelGGL((attn_b_native<FMT, PB_PAIR>), dim3(nB), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((attn_b_native<FMT, PB_PLAIN>), dim3(groups * kblocks), dim3(256), 0, s, a);
  }
}

hipError_t launch_attn_b_native(const AttnArgs &a, hipStream_t s) {
  KernelTimer timer(H2O_K_ATTN_B, s);
  switch (a.cache_fmt) {
    case FMT_INT8: launch_b_fmt<FMT_INT8>(a, s); break;
    case FMT_INT4: launch_b_fmt<FMT_INT4>(a, s); break;
    default: launch_b_fmt<FMT_NATIVE>(a, s); break;
  }
  return hipGetLastError();
}

}  // namespace h2o
