// Per-kernel HIP-event timing behind tcs_timing_enable / tcs_timing_read.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <utility>
#include <vector>

#include "tcs_internal.h"

namespace tcs {
namespace {

using EventPair = std::pair<hipEvent_t, hipEvent_t>;

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<EventPair> g_pool;                   // idle event pairs
std::vector<EventPair> g_done[TCS_TIMER_COUNT];  // recorded, not yet read
thread_local EventPair t_open[TCS_TIMER_COUNT] = {};  // started on this thread

bool take_pair(EventPair* out) {
  {
    std::lock_guard<std::mutex> g(g_mu);
    if (!g_pool.empty()) {
      *out = g_pool.back();
      g_pool.pop_back();
      return true;
    }
  }
  hipEvent_t a = nullptr, b = nullptr;
  if (hipEventCreate(&a) != hipSuccess) return false;
  if (hipEventCreate(&b) != hipSuccess) {
    (void)hipEventDestroy(a);
    return false;
  }
  *out = {a, b};
  return true;
}

void give_back(const EventPair& p) {
  std::lock_guard<std::mutex> g(g_mu);
  g_pool.push_back(p);
}

}  // namespace

void timer_begin(int timer, void* stream) {
  if (!g_on.load(std::memory_order_relaxed) || timer < 0 || timer >= TCS_TIMER_COUNT) return;
  EventPair& o = t_open[timer];
  if (o.first) give_back(o);  // a launch that failed between begin and end
  o = {};
  EventPair p;
  if (!take_pair(&p)) return;
  if (hipEventRecord(p.first, static_cast<hipStream_t>(stream)) != hipSuccess) {
    give_back(p);
    return;
  }
  o = p;
}

void timer_end(int timer, void* stream) {
  if (timer < 0 || timer >= TCS_TIMER_COUNT) return;
  EventPair& o = t_open[timer];
  if (!o.first) return;
  const EventPair p = o;
  o = {};
  if (hipEventRecord(p.second, static_cast<hipStream_t>(stream)) != hipSuccess) {
    give_back(p);
    return;
  }
  std::lock_guard<std::mutex> g(g_mu);
  g_done[timer].push_back(p);
}

}  // namespace tcs

using namespace tcs;

extern "C" int tcs_timing_enable(int enable) {
  clear_error();
  if (enable) {
    g_on.store(true);
    return TCS_OK;
  }
  g_on.store(false);
  std::vector<EventPair> all;
  {
    std::lock_guard<std::mutex> g(g_mu);
    all.swap(g_pool);
    for (auto& v : g_done) {
      all.insert(all.end(), v.begin(), v.end());
      v.clear();
    }
  }
  for (auto& p : all) {
    (void)hipEventSynchronize(p.second);
    (void)hipEventDestroy(p.first);
    (void)hipEventDestroy(p.second);
  }
  return TCS_OK;
}

extern "C" int tcs_timing_read(int timer, double* total_ms, int32_t* launches) {
  clear_error();
  if (timer < 0 || timer >= TCS_TIMER_COUNT || !total_ms || !launches)
    return fail(TCS_EINVAL, "timing_read: timer %d, outputs %p %p", timer, (void*)total_ms,
                (void*)launches);
  std::vector<EventPair> rec;
  {
    std::lock_guard<std::mutex> g(g_mu);
    rec.swap(g_done[timer]);
  }
  double sum = 0.0;
  int status = TCS_OK;
  for (auto& p : rec) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(p.second);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, p.first, p.second);
    if (e != hipSuccess && status == TCS_OK)
      status = fail(TCS_EHIP, "timing_read: %s", hipGetErrorString(e));
    sum += ms;
    give_back(p);
  }
  *total_ms = sum;
  *launches = int32_t(rec.size());
  return status;
}
