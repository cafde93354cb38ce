// Optional kernel timing: while enabled, each kernel launch of the library is
// bracketed by two hipEvents recorded on the caller's stream; reading the
// totals waits for those events.  Events come from a pool owned here (no
// device memory is allocated).

#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "../../include/h2o.h"
#include "h2o_internal.hpp"

namespace h2o {
namespace {

struct Pending {
  hipEvent_t start, stop;
  int kind;
};

std::mutex g_mu;
bool g_enabled = false;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_pool;
double g_total_ms[H2O_K_COUNT] = {};
long long g_launches[H2O_K_COUNT] = {};

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

KernelTimer::KernelTimer(int kind, hipStream_t s) : kind_(kind), stream_(s) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_enabled) return;
  start_ = take_event();
  if (start_ && hipEventRecord(start_, s) != hipSuccess) {
    g_pool.push_back(start_);
    start_ = nullptr;
  }
}

KernelTimer::~KernelTimer() {
  if (!start_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t stop = take_event();
  if (stop && hipEventRecord(stop, stream_) == hipSuccess) {
    g_pending.push_back({start_, stop, kind_});
  } else {
    g_pool.push_back(start_);
    if (stop) g_pool.push_back(stop);
  }
}

}  // namespace h2o

extern "C" {

int h2o_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(h2o::g_mu);
  h2o::g_enabled = on != 0;
  return H2O_OK;
}

int h2o_profile_read(double *total_ms, int64_t *launches, int n) {
  if (!total_ms || !launches || n < H2O_K_COUNT) return H2O_EINVAL;
  std::lock_guard<std::mutex> lk(h2o::g_mu);
  for (const auto &p : h2o::g_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.stop) == hipSuccess &&
        hipEventElapsedTime(&ms, p.start, p.stop) == hipSuccess) {
      h2o::g_total_ms[p.kind] += ms;
      h2o::g_launches[p.kind] += 1;
    }
    h2o::g_pool.push_back(p.start);
    h2o::g_pool.push_back(p.stop);
  }
  h2o::g_pending.clear();
  for (int k = 0; k < H2O_K_COUNT; ++k) {
    total_ms[k] = h2o::g_total_ms[k];
    launches[k] = h2o::g_launches[k];
  }
  return H2O_OK;
}

int h2o_profile_reset(void) {
  std::lock_guard<std::mutex> lk(h2o::g_mu);
  for (const auto &p : h2o::g_pending) {
    hipEventSynchronize(p.stop);
    h2o::g_pool.push_back(p.start);
    h2o::g_pool.push_back(p.stop);
  }
  h2o::g_pending.clear();
  for (int k = 0; k < H2O_K_COUNT; ++k) {
    h2o::g_total_ms[k] = 0.0;
    h2o::g_launches[k] = 0;
  }
  return H2O_OK;
}

}  // extern "C"
