// Opt-in kernel timing: when enabled, the library records a pair of HIP
// events on the launch stream around each of its dominant kernels. Reading
// waits for the recorded events and sums their elapsed times per kind.
#include <atomic>
#include <mutex>
#include <vector>

#include "internal.h"

namespace qnf4 {
namespace {

std::atomic<bool> g_on{false};
std::mutex g_mu;
struct EventPair {
  hipEvent_t start, stop;
};
std::vector<EventPair> g_done[kProfKinds];
thread_local hipEvent_t g_open[kProfKinds] = {};

}  // namespace

bool prof_enabled() { return g_on.load(std::memory_order_relaxed); }

void prof_set(bool on) { g_on.store(on, std::memory_order_relaxed); }

void prof_begin(int kind, hipStream_t s) {
  if (!prof_enabled()) return;
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return;
  (void)hipEventRecord(e, s);
  g_open[kind] = e;
}

void prof_end(int kind, hipStream_t s) {
  if (!prof_enabled() || !g_open[kind]) return;
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return;
  (void)hipEventRecord(e, s);
  std::lock_guard<std::mutex> lk(g_mu);
  g_done[kind].push_back({g_open[kind], e});
  g_open[kind] = nullptr;
}

hipError_t prof_read(int kind, double *total_ms, int64_t *count) {
  std::lock_guard<std::mutex> lk(g_mu);
  double sum = 0.0;
  for (const EventPair &p : g_done[kind]) {
    hipError_t err = hipEventSynchronize(p.stop);
    if (err != hipSuccess) return err;
    float ms = 0.0f;
    err = hipEventElapsedTime(&ms, p.start, p.stop);
    if (err != hipSuccess) return err;
    sum += ms;
  }
  *total_ms = sum;
  *count = static_cast<int64_t>(g_done[kind].size());
  return hipSuccess;
}

void prof_reset() {
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto &v : g_done) {
    for (const EventPair &p : v) {
      (void)hipEventSynchronize(p.stop);
      (void)hipEventDestroy(p.start);
      (void)hipEventDestroy(p.stop);
    }
    v.clear();
  }
}

}  // namespace qnf4
