// Host-side checker of the C ABI's argument validation, built with
// AddressSanitizer on the host code of the ABI layer (the debug build).  It
// calls every entry point with arguments that validation must reject and
// checks the status codes; no call gets past validation, so no kernel runs
// and no GPU is needed.  Prints "abi checks ok" and exits 0 on success.

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/h2o.h"

// From the HIP runtime (the checker refuses to run where a GPU is visible,
// so that a validation gap can never launch a kernel on fake addresses).
extern "C" int hipGetDeviceCount(int *count);

namespace {

int failures = 0;

void expect(int got, int want, const char *what) {
  if (got != want) {
    std::printf("FAIL %s: got %d want %d\n", what, got, want);
    ++failures;
  }
}

h2o_dims dims(int B, int Hq, int Hkv, int D, int C, int T, int fmt = H2O_CACHE_NATIVE, int dtype = H2O_BF16) {
  h2o_dims d;
  std::memset(&d, 0, sizeof(d));
  d.B = B;
  d.Hq = Hq;
  d.Hkv = Hkv;
  d.D = D;
  d.C = C;
  d.T = T;
  d.dtype = dtype;
  d.cache_fmt = fmt;
  d.policy = H2O_POLICY_H2O;
  d.scale = 0.f;
  return d;
}

}  // namespace

int main() {
  int devices = 0;
  if (hipGetDeviceCount(&devices) == 0 && devices > 0) {
    std::printf("a GPU is visible: this checker runs on hosts without one\n");
    return 2;
  }
  // a fake, 16-byte aligned address that validation never lets a kernel see
  void *F = reinterpret_cast<void *>(static_cast<uintptr_t>(0x10000));
  float *Ff = static_cast<float *>(F);
  int32_t *Fi = static_cast<int32_t *>(F);
  uint16_t *Fh = static_cast<uint16_t *>(F);
  h2o_cache cache = {F, F, Fh, Fh, Fh, Fh, Ff, Fi};

  expect(h2o_abi_version(), H2O_ABI_VERSION, "abi version");
  for (int s = -8; s <= 8; ++s) {
    const char *str = h2o_status_str(s);
    if (!str || !std::strlen(str)) {
      std::printf("FAIL status string %d\n", s);
      ++failures;
    }
  }

  // workspace sizes over a grid of shapes: valid ones positive, invalid zero
  const int Ds[] = {32, 64, 96, 128};
  const int Cs[] = {1, 63, 64, 4096, 65536, (1 << 22) - 64, 1 << 22};
  const int Ts[] = {1, 4, 16, 64, 1024};
  for (int D : Ds)
    for (int C : Cs)
      for (int T : Ts)
        for (int fmt = 0; fmt < 3; ++fmt) {
          h2o_dims d = dims(1, 32, 8, D, C, T, fmt);
          const size_t nb = h2o_workspace_bytes(&d);
          const bool valid = (D == 64 || D == 128) && static_cast<long long>(C) + T <= (1 << 22);
          if (valid != (nb > 0)) {
            std::printf("FAIL workspace D=%d C=%d T=%d fmt=%d: %zu\n", D, C, T, fmt, nb);
            ++failures;
          }
        }
  expect(static_cast<int>(h2o_workspace_bytes(nullptr)), 0, "workspace of null dims");

  h2o_dims d = dims(1, 8, 2, 128, 256, 64);
  const size_t ws_bytes = h2o_workspace_bytes(&d);
  // attention
  expect(h2o_sdpa_scoresum(nullptr, &cache, 0, F, F, F, F, Ff, nullptr, F, ws_bytes, nullptr), H2O_EINVAL,
         "sdpa null dims");
  expect(h2o_sdpa_scoresum(&d, &cache, 0, nullptr, F, F, F, Ff, nullptr, F, ws_bytes, nullptr), H2O_EINVAL,
         "sdpa null q");
  expect(h2o_sdpa_scoresum(&d, &cache, 257, F, F, F, F, Ff, nullptr, F, ws_bytes, nullptr), H2O_EINVAL,
         "sdpa n_occ > C");
  expect(h2o_sdpa_scoresum(&d, &cache, 0, F, F, F, F, Ff, nullptr, F, 16, nullptr), H2O_EWORKSPACE,
         "sdpa small workspace");
  expect(h2o_sdpa_scoresum(&d, &cache, 0, static_cast<char *>(F) + 4, F, F, F, Ff, nullptr, F, ws_bytes, nullptr),
         H2O_EINVAL, "sdpa misaligned q");
  h2o_dims bad = dims(1, 8, 3, 128, 256, 64);
  expect(h2o_sdpa_scoresum(&bad, &cache, 0, F, F, F, F, Ff, nullptr, F, ws_bytes, nullptr), H2O_EINVAL,
         "sdpa Hq % Hkv");
  bad = dims(1, 8, 2, 96, 256, 64);
  expect(h2o_sdpa_scoresum(&bad, &cache, 0, F, F, F, F, Ff, nullptr, F, ws_bytes, nullptr), H2O_EUNSUPPORTED,
         "sdpa D=96");
  bad = dims(1024, 8, 8, 128, 1 << 18, 64);
  expect(h2o_sdpa_scoresum(&bad, &cache, 0, F, F, F, F, Ff, nullptr, F, ws_bytes, nullptr), H2O_EUNSUPPORTED,
         "sdpa past 32-bit indices");
  // selection
  expect(h2o_evict_topk(&d, &cache, 200, 0, Ff, Fi, nullptr, 0, nullptr), H2O_EUNSUPPORTED, "evict straddle");
  expect(h2o_evict_topk(&d, &cache, 0, -1, Ff, Fi, nullptr, 0, nullptr), H2O_EINVAL, "evict negative pos");
  h2o_cache no_scores = cache;
  no_scores.scores = nullptr;
  expect(h2o_evict_topk(&d, &no_scores, 0, 0, Ff, Fi, nullptr, 0, nullptr), H2O_EINVAL, "evict no scores");
  h2o_dims norm = d;
  norm.policy = H2O_POLICY_NORM;
  h2o_cache no_pos = cache;
  no_pos.token_pos = nullptr;
  expect(h2o_evict_topk(&norm, &no_pos, 0, 0, Ff, Fi, nullptr, 0, nullptr), H2O_EINVAL, "h2o_norm without positions");
  expect(h2o_evict_topk(&d, &cache, 0, 0, Ff, Fi, static_cast<char *>(F) + 8, 64, nullptr), H2O_EWORKSPACE,
         "evict misaligned workspace");
  // writes
  expect(kv_scatter(&d, &cache, F, F, nullptr, nullptr), H2O_EINVAL, "scatter null log");
  expect(kv_quant_pack(&d, &cache, F, F, Fi, nullptr), H2O_EINVAL, "quant pack on a native cache");
  h2o_dims i4 = dims(1, 8, 2, 128, 256, 64, H2O_CACHE_INT4);
  h2o_cache no_zero = cache;
  no_zero.k_zero = nullptr;
  expect(kv_quant_pack(&i4, &no_zero, F, F, Fi, nullptr), H2O_EINVAL, "int4 pack without zero points");
  expect(kv_dequant_unpack(&d, &cache, 0, Ff, Ff, nullptr), H2O_EINVAL, "unpack zero slots");
  // whole step, no-allocation step, replay
  expect(h2o_chunk_step(&d, &cache, 0, 0, F, F, F, F, Ff, Fi, F, 16, nullptr), H2O_EWORKSPACE, "step workspace");
  expect(h2o_chunk_step(&d, &cache, -1, 0, F, F, F, F, Ff, Fi, F, ws_bytes, nullptr), H2O_EINVAL,
         "step n_occ < 0");
  expect(h2o_chunk_step_noalloc(&d, &cache, 300, 0, F, F, F, F, Ff, Fi, nullptr), H2O_EINVAL, "noalloc n_occ > C");
  h2o_dims big = dims(1, 32, 8, 128, 1 << 20, 4);
  expect(h2o_chunk_step_noalloc(&big, &cache, 1 << 20, 0, F, F, F, F, nullptr, Fi, nullptr), H2O_EWORKSPACE,
         "noalloc workspace beyond the array");
  expect(h2o_replay_step(&d, &cache, 200, 0, F, F, F, F, Fi, F, ws_bytes, nullptr), H2O_EUNSUPPORTED,
         "replay straddle");
  // backward
  h2o_dims i8 = dims(1, 8, 2, 128, 256, 64, H2O_CACHE_INT8);
  expect(h2o_sdpa_backward(&i8, &cache, 0, F, F, F, Ff, F, Ff, Ff, Ff, Ff, Ff, F, ws_bytes, nullptr),
         H2O_EUNSUPPORTED, "backward on an int8 cache");
  expect(h2o_sdpa_backward(&d, &cache, 10, F, F, F, Ff, F, Ff, nullptr, Ff, Ff, Ff, F, ws_bytes, nullptr),
         H2O_EINVAL, "backward without cache gradients");
  expect(h2o_sdpa_backward(&d, &cache, 0, F, F, F, Ff, F, Ff, Ff, Ff, Ff, Ff, F, 8, nullptr), H2O_EWORKSPACE,
         "backward workspace");
  // timers: too few entries
  std::vector<double> ms(2);
  std::vector<int64_t> cnt(2);
  expect(h2o_profile_read(ms.data(), cnt.data(), 2), H2O_EINVAL, "profile read with short arrays");

  if (failures) {
    std::printf("%d abi checks failed\n", failures);
    return 1;
  }
  std::printf("abi checks ok\n");
  return 0;
}
