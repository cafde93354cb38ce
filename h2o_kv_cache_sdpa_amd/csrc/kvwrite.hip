// Slot overwrite for the cache buffers.
//
// Native: copy each new key/value row into its slot ("Learning how to
// Forget", §A.8: scatter along the slot axis, head dimension contiguous) as
// 16-byte chunks, consecutive threads on consecutive chunks of a row.
//
// Quantised: one wavefront per row quantises and writes codes plus fp16 scale
// (and zero point), with the per-slot scheme of kv_quant.hpp.

#include "device_util.hpp"
#include "h2o_internal.hpp"
#include "kv_quant.hpp"

namespace h2o {
namespace {

__global__ __launch_bounds__(256) void scatter_native(KvWriteArgs a, int row_bytes) {
  const int cpr = row_bytes / 16;
  const size_t rows = static_cast<size_t>(a.groups) * a.T;
  const size_t c = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (c >= rows * cpr) return;
  const int isv = blockIdx.y;
  const size_t r = c / cpr;
  const int chunk = static_cast<int>(c % cpr);
  const int grp = static_cast<int>(r / a.T);
  const int slot = a.slot_log[r];
  if (slot < 0 || slot >= a.C) return;  // caller-supplied log: never write outside the cache
  if (a.token_pos && chunk == 0 && isv == 0)
    a.token_pos[static_cast<size_t>(grp) * a.C + slot] = static_cast<int32_t>(a.pos + static_cast<int>(r % a.T));
  H2O_DEVICE_CHECK(grp < a.groups && chunk < cpr);
  const char *src = static_cast<const char *>(isv ? a.vn : a.kn) + r * row_bytes + chunk * 16;
  char *dst = static_cast<char *>(isv ? a.vc : a.kc) +
              (static_cast<size_t>(grp) * a.C + slot) * row_bytes + chunk * 16;
  *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
}

// One wavefront per row; lane l handles elements 2l and 2l+1 (D <= 128).
template <int DT, int FMT>
__global__ __launch_bounds__(256) void quant_pack(KvWriteArgs a) {
  const int lane = threadIdx.x & 63;
  const size_t nrows = static_cast<size_t>(a.groups) * a.T;
  const size_t r = static_cast<size_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= 2 * nrows) return;
  const bool isv = r >= nrows;
  const size_t rr = isv ? r - nrows : r;
  const int grp = static_cast<int>(rr / a.T);
  const int slot = a.slot_log[rr];
  if (slot < 0 || slot >= a.C) return;  // wave-uniform: one row per wavefront
  const size_t dst_row = static_cast<size_t>(grp) * a.C + slot;
  if (a.token_pos && !isv && lane == 0) a.token_pos[dst_row] = static_cast<int32_t>(a.pos + static_cast<int>(rr % a.T));
  quantize_row<DT, FMT>(a, rr, dst_row, isv, lane);
}

template <int DT, int FMT>
__global__ __launch_bounds__(256) void dequant_rows(KvWriteArgs a, int n_slots, float *kout,
                                                    float *vout) {
  const size_t n = static_cast<size_t>(a.groups) * n_slots * a.D;
  const size_t e = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= n) return;
  const int d = static_cast<int>(e % a.D);
  const size_t rs = e / a.D;  // grp * n_slots + slot
  const int slot = static_cast<int>(rs % n_slots);
  const size_t grp = rs / n_slots;
  const size_t row = grp * a.C + slot;
  const void *buf = blockIdx.y ? a.vc : a.kc;
  const uint16_t *sc = blockIdx.y ? a.vs : a.ks;
  const uint16_t *zr = blockIdx.y ? a.vz : a.kz;
  (blockIdx.y ? vout : kout)[e] = cache_elem<DT, FMT>(buf, sc, zr, row, d, a.D);
}

template <int DT>
hipError_t launch_quant_dt(const KvWriteArgs &a, hipStream_t s) {
  const size_t rows = 2 * static_cast<size_t>(a.groups) * a.T;
  const dim3 grid(static_cast<unsigned>((rows + 3) / 4));
  if (a.cache_fmt == FMT_INT8) {
    hipLaunchKernelGGL((quant_pack<DT, FMT_INT8>), grid, dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((quant_pack<DT, FMT_INT4>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

template <int DT, int FMT>
hipError_t launch_dequant_t(const KvWriteArgs &a, int n_slots, float *kout, float *vout,
                            hipStream_t s) {
  const size_t n = static_cast<size_t>(a.groups) * n_slots * a.D;
  const dim3 grid(static_cast<unsigned>((n + 255) / 256), 2);
  hipLaunchKernelGGL((dequant_rows<DT, FMT>), grid, dim3(256), 0, s, a, n_slots, kout, vout);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dequant_dt(const KvWriteArgs &a, int n_slots, float *kout, float *vout,
                             hipStream_t s) {
  switch (a.cache_fmt) {
    case FMT_INT8: return launch_dequant_t<DT, FMT_INT8>(a, n_slots, kout, vout, s);
    case FMT_INT4: return launch_dequant_t<DT, FMT_INT4>(a, n_slots, kout, vout, s);
    default: return launch_dequant_t<DT, FMT_NATIVE>(a, n_slots, kout, vout, s);
  }
}

}  // namespace

hipError_t launch_kv_write(const KvWriteArgs &a, hipStream_t s) {
  KernelTimer timer(H2O_K_KV_WRITE, s);
  if (a.cache_fmt == FMT_NATIVE) {
    const int row_bytes = a.D * (a.dtype == DT_F32 ? 4 : 2);
    const size_t chunks = static_cast<size_t>(a.groups) * a.T * (row_bytes / 16);
    const dim3 grid(static_cast<unsigned>((chunks + 255) / 256), 2);
    hipLaunchKernelGGL(scatter_native, grid, dim3(256), 0, s, a, row_bytes);
    return hipGetLastError();
  }
  if (a.dtype == DT_F32) return launch_quant_dt<DT_F32>(a, s);
  return launch_quant_dt<DT_BF16>(a, s);
}

hipError_t launch_dequant(const KvWriteArgs &a, int n_slots, float *kout, float *vout,
                          hipStream_t s) {
  if (a.dtype == DT_F32) return launch_dequant_dt<DT_F32>(a, n_slots, kout, vout, s);
  return launch_dequant_dt<DT_BF16>(a, n_slots, kout, vout, s);
}

}  // namespace h2o
