// Optional per-launch timing of the hot calls (diagnostics).  When enabled,
// every kernel launch is bracketed by a pair of HIP events recorded on the
// launch's own stream; the caller reads the durations after synchronising.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/fpd.h"
#include "kernels.h"

namespace fpd {
namespace {

struct Rec {
  const char* tag;
  hipEvent_t a, b;
};

std::mutex g_mu;                  // guards the records and the event pool
std::atomic<bool> g_on{false};    // read without the lock on every launch
thread_local int t_quiet = 0;     // NoTiming scopes alive on this thread
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;  // events kept for reuse until the process ends

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

void recycle_all() {
  for (Rec& r : g_recs) {
    if (r.a) g_pool.push_back(r.a);
    if (r.b) g_pool.push_back(r.b);
  }
  g_recs.clear();
}

}  // namespace

ProfScope::ProfScope(const char* tag, hipStream_t st) : st_(st), idx_(-1) {
  if (!g_on.load(std::memory_order_relaxed) || t_quiet > 0) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on.load(std::memory_order_relaxed)) return;
  Rec r{tag, take_event(), take_event()};
  if (!r.a || !r.b) return;
  if (hipEventRecord(r.a, st) != hipSuccess) return;
  idx_ = (int)g_recs.size();
  g_recs.push_back(r);
}

ProfScope::~ProfScope() {
  if (idx_ < 0) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (idx_ < (int)g_recs.size()) (void)hipEventRecord(g_recs[idx_].b, st_);
}

NoTiming::NoTiming() { ++t_quiet; }
NoTiming::~NoTiming() { --t_quiet; }

}  // namespace fpd

using namespace fpd;

extern "C" {

int32_t fpd_profile_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_mu);
  recycle_all();
  g_on.store(on != 0, std::memory_order_relaxed);
  return FPD_OK;
}

int32_t fpd_profile_count(int32_t* n) {
  if (!n) return FPD_E_ARG;
  std::lock_guard<std::mutex> lk(g_mu);
  *n = (int32_t)g_recs.size();
  return FPD_OK;
}

int32_t fpd_profile_read(int32_t i, const char** tag, float* ms) {
  if (!tag || !ms) return FPD_E_ARG;
  std::lock_guard<std::mutex> lk(g_mu);
  if (i < 0 || i >= (int32_t)g_recs.size()) return FPD_E_ARG;
  *tag = g_recs[i].tag;
  const hipError_t e = hipEventElapsedTime(ms, g_recs[i].a, g_recs[i].b);
  return e == hipSuccess ? FPD_OK : FPD_E_HIP;
}

}  // extern "C"
