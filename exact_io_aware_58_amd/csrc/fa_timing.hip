// fa_timing.hip -- optional per-kernel device timing with hipEvents recorded
// on the launch stream around each kernel.  Host-only code.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "../../include/fa.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kPool = 8192;

struct Pending {
  int id;
  int slot;
};

struct Timer {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> start, stop;
  int next = 0;      // next unused event slot
  int in_flight = 0;  // slots taken by launches whose stop event is not yet recorded
  std::vector<Pending> pending;
  long long launches[FA_KERNEL_COUNT] = {};
  double total_ms[FA_KERNEL_COUNT] = {};
  long long dropped = 0;
};

Timer& timer() {
  static Timer t;
  return t;
}

// Sum every pending pair into the totals.  Caller holds the mutex.
int drain(Timer& t) {
  for (const Pending& p : t.pending) {
    if (hipEventSynchronize(t.stop[p.slot]) != hipSuccess) return FA_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, t.start[p.slot], t.stop[p.slot]) != hipSuccess) return FA_ERR_HIP;
    t.launches[p.id] += 1;
    t.total_ms[p.id] += ms;
  }
  t.pending.clear();
  // Slots are reused only when no launch still holds one between its two
  // events (another thread may be inside a timed launch).
  if (t.in_flight == 0) t.next = 0;
  return FA_OK;
}

}  // namespace

TimedLaunch::TimedLaunch(int kernel_id, hipStream_t s) : id(kernel_id), stream(s), slot(-1) {
  Timer& t = timer();
  std::lock_guard<std::mutex> g(t.mu);
  if (!t.on) return;
  if (t.next >= kPool) {
    t.dropped += 1;
    return;
  }
  slot = t.next++;
  if (hipEventRecord(t.start[slot], stream) != hipSuccess)
    slot = -1;
  else
    t.in_flight += 1;
}

TimedLaunch::~TimedLaunch() {
  if (slot < 0) return;
  Timer& t = timer();
  std::lock_guard<std::mutex> g(t.mu);
  t.in_flight -= 1;
  if (hipEventRecord(t.stop[slot], stream) == hipSuccess) t.pending.push_back({id, slot});
}

}  // namespace fa

extern "C" int fa_timing_enable(int on) {
  fa::Timer& t = fa::timer();
  std::lock_guard<std::mutex> g(t.mu);
  if (on) {
    if (t.start.empty()) {
      t.start.resize(fa::kPool);
      t.stop.resize(fa::kPool);
      for (int i = 0; i < fa::kPool; ++i) {
        if (hipEventCreate(&t.start[i]) != hipSuccess || hipEventCreate(&t.stop[i]) != hipSuccess)
          return FA_ERR_HIP;
      }
    }
    int rc = fa::drain(t);
    for (int k = 0; k < FA_KERNEL_COUNT; ++k) {
      t.launches[k] = 0;
      t.total_ms[k] = 0.0;
    }
    t.dropped = 0;
    t.on = true;
    return rc;
  }
  int rc = fa::drain(t);
  t.on = false;
  return rc;
}

extern "C" int fa_timing_read(int kernel_id, long long* launches, double* total_ms,
                              long long* dropped) {
  if (kernel_id < 0 || kernel_id >= FA_KERNEL_COUNT || !launches || !total_ms)
    return FA_ERR_INVALID_ARG;
  fa::Timer& t = fa::timer();
  std::lock_guard<std::mutex> g(t.mu);
  int rc = fa::drain(t);
  *launches = t.launches[kernel_id];
  *total_ms = t.total_ms[kernel_id];
  if (dropped) *dropped = t.dropped;
  return rc;
}

extern "C" const char* fa_kernel_name(int kernel_id) {
  switch (kernel_id) {
    case FA_KERNEL_FWD: return "fwd";
    case FA_KERNEL_BWD_DELTA: return "bwd_delta";
    case FA_KERNEL_BWD_DKDV: return "bwd_dkdv";
    case FA_KERNEL_BWD_DQ: return "bwd_dq";
    case FA_KERNEL_MERGE: return "merge";
    case FA_KERNEL_BWD_DKDV_DQ: return "bwd_dkdv_dq";
    default: return "unknown";
  }
}
