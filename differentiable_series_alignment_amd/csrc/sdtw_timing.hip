// Optional launch timing: HIP events recorded on the caller's stream around
// every kernel the library enqueues (sdtw_timing / sdtw_timing_collect in
// include/sdtw.h).  Off by default; one record list per process, guarded by
// a mutex (frameworks may issue the backward from another host thread).
#include <atomic>
#include <mutex>
#include <vector>

#include "sdtw.h"
#include "sdtw_kernels.h"

namespace sdtw {
namespace {

struct TimingRecord {
  const char* name;
  hipEvent_t begin, end;
  bool closed;  // the end event has been recorded
};

struct TimingState {
  std::atomic<bool> on{false};
  std::mutex lock;
  std::vector<TimingRecord> records;
};

TimingState g_timing;
thread_local int t_no_timing = 0;

}  // namespace

NoTimingScope::NoTimingScope() { ++t_no_timing; }
NoTimingScope::~NoTimingScope() { --t_no_timing; }

TimedLaunch::TimedLaunch(const char* name, hipStream_t s) : stream_(s), index_(-1) {
  if (!g_timing.on || t_no_timing) return;
  TimingRecord r{name, nullptr, nullptr, false};
  if (hipEventCreate(&r.begin) != hipSuccess) return;
  if (hipEventCreate(&r.end) != hipSuccess) {
    (void)hipEventDestroy(r.begin);
    return;
  }
  if (hipEventRecord(r.begin, s) != hipSuccess) {
    (void)hipEventDestroy(r.begin);
    (void)hipEventDestroy(r.end);
    return;
  }
  std::lock_guard<std::mutex> g(g_timing.lock);
  g_timing.records.push_back(r);
  index_ = 0;
  end_ = r.end;
}

TimedLaunch::~TimedLaunch() {
  if (index_ < 0) return;
  std::lock_guard<std::mutex> g(g_timing.lock);
  (void)hipEventRecord(end_, stream_);
  for (TimingRecord& r : g_timing.records)
    if (r.end == end_) r.closed = true;
}

}  // namespace sdtw

extern "C" {

int sdtw_timing(int on) {
  sdtw::g_timing.on = on != 0;
  return SDTW_OK;
}

int sdtw_timing_collect(const char** names, float* ms, int cap) {
  std::lock_guard<std::mutex> g(sdtw::g_timing.lock);
  int n = 0;
  bool failed = false;
  std::vector<sdtw::TimingRecord> open;
  for (const sdtw::TimingRecord& r : sdtw::g_timing.records) {
    if (!r.closed) {
      open.push_back(r);
      continue;
    }
    float t = -1.f;
    if (hipEventSynchronize(r.end) != hipSuccess ||
        hipEventElapsedTime(&t, r.begin, r.end) != hipSuccess)
      failed = true;
    if (n < cap && names && ms) {
      names[n] = r.name;
      ms[n] = t;
    }
    ++n;
    (void)hipEventDestroy(r.begin);
    (void)hipEventDestroy(r.end);
  }
  sdtw::g_timing.records.swap(open);
  return failed ? -SDTW_ERR_HIP : n;
}

}  // extern "C"
