// Per-kernel timing with HIP events, for benchmarks (msr_trace_* in msr.h).
// When enabled, every launcher brackets its kernel with an event pair
// recorded on the launch stream; msr_trace_count() waits for the recorded
// events and folds them into per-kernel totals.  Diagnostics only: the state
// below is process-wide and not thread safe.
#include <map>
#include <string>
#include <utility>
#include <vector>

#include "../../include/msr.h"
#include "msr_launch.h"

namespace msr {
namespace {
struct Pending {
  const char* name;
  hipEvent_t start, stop;
};
bool g_on = false;
std::vector<Pending> g_pending;
std::map<std::string, std::pair<double, int64_t>> g_totals;
std::vector<std::pair<std::string, std::pair<double, int64_t>>> g_snapshot;

void drain() {
  for (auto& p : g_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.stop) == hipSuccess && hipEventElapsedTime(&ms, p.start, p.stop) == hipSuccess) {
      auto& t = g_totals[p.name];
      t.first += ms;
      t.second += 1;
    }
    (void)hipEventDestroy(p.start);
    (void)hipEventDestroy(p.stop);
  }
  g_pending.clear();
}
}  // namespace

TraceScope::TraceScope(const char* name, hipStream_t stream) : name_(name), stream_(stream) {
  if (!g_on) return;
  if (hipEventCreate(&start_) != hipSuccess) return;
  if (hipEventCreate(&stop_) != hipSuccess) {
    (void)hipEventDestroy(start_);
    return;
  }
  active_ = hipEventRecord(start_, stream_) == hipSuccess;
  if (!active_) {
    (void)hipEventDestroy(start_);
    (void)hipEventDestroy(stop_);
  }
}

TraceScope::~TraceScope() {
  if (!active_) return;
  if (hipEventRecord(stop_, stream_) == hipSuccess) {
    g_pending.push_back({name_, start_, stop_});
  } else {
    (void)hipEventDestroy(start_);
    (void)hipEventDestroy(stop_);
  }
}

}  // namespace msr

extern "C" {

void msr_trace_enable(int32_t on) {
  using namespace msr;
  drain();
  g_totals.clear();
  g_snapshot.clear();
  g_on = on != 0;
}

int32_t msr_trace_count(void) {
  using namespace msr;
  drain();
  g_snapshot.assign(g_totals.begin(), g_totals.end());
  return (int32_t)g_snapshot.size();
}

msr_status msr_trace_get(int32_t i, const char** name, double* total_ms, int64_t* launches) {
  using namespace msr;
  if (i < 0 || i >= (int32_t)g_snapshot.size()) return MSR_ERR_SHAPE;
  if (name) *name = g_snapshot[i].first.c_str();
  if (total_ms) *total_ms = g_snapshot[i].second.first;
  if (launches) *launches = g_snapshot[i].second.second;
  return MSR_OK;
}

}  // extern "C"
