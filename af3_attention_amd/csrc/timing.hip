// Per-kernel timing with HIP events recorded on the launch stream (profiling
// aid; see evoattn_timing_enable in include/evoattn.h).

#include <atomic>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "evoattn.h"
#include "evoattn_internal.h"

namespace {

struct Pending {
  std::string name;
  hipEvent_t start;
  hipEvent_t stop;
};

std::atomic<int> g_enabled{0};
std::mutex g_mu;
std::vector<Pending> g_pending;

}  // namespace

namespace evo {

KernelTimer::KernelTimer(const char* name, hipStream_t stream) : name_(name), stream_(stream) {
  if (!g_enabled.load(std::memory_order_relaxed)) return;
  if (hipEventCreate(&start_) != hipSuccess) {
    start_ = nullptr;
    return;
  }
  if (hipEventRecord(start_, stream_) != hipSuccess) {
    (void)hipEventDestroy(start_);
    start_ = nullptr;
  }
}

KernelTimer::~KernelTimer() {
  if (!start_) return;
  hipEvent_t stop = nullptr;
  if (hipEventCreate(&stop) != hipSuccess || hipEventRecord(stop, stream_) != hipSuccess) {
    if (stop) (void)hipEventDestroy(stop);
    (void)hipEventDestroy(start_);
    return;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  g_pending.push_back({name_, start_, stop});
}

}  // namespace evo

extern "C" {

void evoattn_timing_enable(int enable) { g_enabled.store(enable ? 1 : 0); }

int evoattn_timing_collect(int max_entries, char* names, int64_t* counts, double* total_ms) {
  std::vector<Pending> pending;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    pending.swap(g_pending);
  }
  std::map<std::string, std::pair<int64_t, double>> agg;
  bool ok = true;
  for (auto& p : pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.stop) != hipSuccess || hipEventElapsedTime(&ms, p.start, p.stop) != hipSuccess)
      ok = false;
    auto& slot = agg[p.name];
    slot.first += 1;
    slot.second += ms;
    (void)hipEventDestroy(p.start);
    (void)hipEventDestroy(p.stop);
  }
  if (!ok) return -1;
  int i = 0;
  for (auto& kv : agg) {
    if (i < max_entries) {
      if (names) {
        std::strncpy(names + 64 * i, kv.first.c_str(), 63);
        names[64 * i + 63] = '\0';
      }
      if (counts) counts[i] = kv.second.first;
      if (total_ms) total_ms[i] = kv.second.second;
    }
    ++i;
  }
  return static_cast<int>(agg.size());
}

}  // extern "C"
