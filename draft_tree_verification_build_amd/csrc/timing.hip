// Kernel timing: per-kernel launch counts and HIP-event durations, for measurement.
//
// While timing is on (dtv_kernel_timing(1)), every launch of the library records one HIP
// event before and one after it on the launch's stream (DTV_LAUNCH in dtv_internal.h). The
// events are kept pending until dtv_kernel_times() reads them: it waits for each pair,
// adds its elapsed time to the kernel's total and returns the pairs' events to a pool for
// reuse. Kernel names are the launched function's name without template arguments.
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "dtv.h"
#include "dtv_internal.h"

namespace {

struct Pending {
  const char* name;
  hipEvent_t begin, end;
};

struct Total {
  std::string name;
  double ms = 0.0;
  long long launches = 0;
};

std::mutex g_mu;
std::atomic<bool> g_on{false};
std::vector<hipEvent_t> g_pool;
std::vector<Pending> g_pending;
std::vector<Total> g_totals;

hipEvent_t take_event() {   // caller holds g_mu
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  // timing only: no system-scope fence (cache writeback and invalidation) when the event
  // completes, which would add its cost to the measured launch and to the next one
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

// "(attn_combine_rows_kernel<128, 8>)" -> "attn_combine_rows_kernel"
std::string base_name(const char* s) {
  std::string out;
  for (const char* p = s; *p; ++p) {
    if (*p == '(' || *p == ' ') continue;
    if (*p == '<' || *p == ')' || *p == ',') break;
    out.push_back(*p);
  }
  return out;
}

// Waits for every pending pair and folds it into the totals (caller holds g_mu).
int resolve_pending() {
  int rc = DTV_OK;
  for (const Pending& p : g_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.end) != hipSuccess || hipEventElapsedTime(&ms, p.begin, p.end) != hipSuccess) {
      rc = DTV_EHIP;
    } else {
      const std::string nm = base_name(p.name);
      Total* t = nullptr;
      for (Total& x : g_totals)
        if (x.name == nm) t = &x;
      if (t == nullptr) {
        g_totals.push_back(Total{nm});
        t = &g_totals.back();
      }
      t->ms += ms;
      t->launches += 1;
    }
    g_pool.push_back(p.begin);
    g_pool.push_back(p.end);
  }
  g_pending.clear();
  return rc;
}

}  // namespace

namespace dtv {

LaunchTimer::LaunchTimer(const char* kernel, hipStream_t stream) : name_(kernel), stream_(stream) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lock(g_mu);
  begin_ = take_event();
  if (begin_ != nullptr && hipEventRecord(begin_, stream_) != hipSuccess) {
    g_pool.push_back(begin_);
    begin_ = nullptr;
  }
}

LaunchTimer::~LaunchTimer() {
  if (begin_ == nullptr) return;
  std::lock_guard<std::mutex> lock(g_mu);
  hipEvent_t end = take_event();
  if (end == nullptr || hipEventRecord(end, stream_) != hipSuccess) {
    g_pool.push_back(begin_);
    if (end != nullptr) g_pool.push_back(end);
    return;
  }
  g_pending.push_back(Pending{name_, begin_, end});
}

}  // namespace dtv

extern "C" {

int dtv_kernel_timing(int enable, int reset) {
  std::lock_guard<std::mutex> lock(g_mu);
  int rc = DTV_OK;
  if (reset) {
    rc = resolve_pending();
    g_totals.clear();
  }
  g_on.store(enable != 0);
  return rc;
}

int dtv_kernel_times(int32_t cap, char* names_h, int32_t name_bytes, double* total_ms_h, int64_t* launches_h) {
  std::lock_guard<std::mutex> lock(g_mu);
  const int rc = resolve_pending();
  if (rc != DTV_OK) return rc;
  const int n = static_cast<int>(g_totals.size());
  for (int i = 0; i < n && i < cap; ++i) {
    if (names_h != nullptr && name_bytes > 0) {
      char* dst = names_h + static_cast<size_t>(i) * name_bytes;
      snprintf(dst, static_cast<size_t>(name_bytes), "%s", g_totals[i].name.c_str());
    }
    if (total_ms_h) total_ms_h[i] = g_totals[i].ms;
    if (launches_h) launches_h[i] = g_totals[i].launches;
  }
  return n;
}

}  // extern "C"
