// fa_launch.h -- host-side interface between the C ABI (fa_api.hip) and the
// kernel launchers.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include <atomic>

namespace fa {

enum Dtype { kF32 = 0, kBF16 = 1, kF16 = 2 };

struct FwdArgs {
  int dtype, B, H;
  int Nq, Nk;  // query rows and key rows per head
  int D;
  int delta;   // causal: key j is visible to query i iff j <= i + delta
  float scale;
  int causal;
  const void *Q, *K, *V;
  void* O;
  float* LSE;
  hipStream_t stream;
};

struct BwdArgs {
  int dtype, B, H, N, D;
  float scale;
  int causal;
  const void *Q, *K, *V, *O, *dO;
  const float* LSE;
  void *dQ, *dK, *dV;
  float* ndelta;  // [B, H, N] float32 in the caller's workspace: -dO_i . O_i
  float* nlse;    // [B, H, N] float32 in the caller's workspace: -LSE_i / scale
  hipStream_t stream;
};

struct MergeArgs {
  int dtype, B, H, N, D;
  void* O;           // [B, H, N, D], partial a on entry, merged result on exit
  float* LSE;        // [B, H, N]
  const void* Ob;    // partial b
  const float* LSEb;
  hipStream_t stream;
};

// Compute units of the current device (queried once per device; 256 on an
// MI355X, used if the query fails).
inline int cu_count() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Causal grids with at most 16 tiles per head and more workgroups than two
// per compute unit take their tiles in tile-major order (see tile_of):
// measured on the B=8, H=12, N=1024 causal step, forward 36.2 -> 27.5 us and
// backward 94.7 -> 76.7 us; long sequences keep the head-major order (no
// change at N=65536).
inline int tile_major(bool causal, int tiles_per_head, long total) {
  return causal && tiles_per_head <= 16 && total > 2L * cu_count() ? 1 : 0;
}

hipError_t launch_fwd(const FwdArgs& a);
hipError_t launch_merge(const MergeArgs& a);
// Each backward launcher enqueues one kernel.
hipError_t launch_bwd_delta(const BwdArgs& a);
hipError_t launch_bwd_dkdv(const BwdArgs& a);
hipError_t launch_bwd_dq(const BwdArgs& a);
// dK/dV at D = 128 without a mask (fa_bwd_d128.hip, its own compile flags).
hipError_t launch_bwd_dkdv_d128_nomask(const BwdArgs& a);
// D = 64 grids of a few rounds: dK/dV and dQ in one launch (fa_bwd.hip).
bool bwd_combined(const BwdArgs& a);
hipError_t launch_bwd_dkdv_dq(const BwdArgs& a);

// Optional per-kernel event timing (fa_timing.cpp).  No-ops when disabled.
struct TimedLaunch {
  TimedLaunch(int kernel_id, hipStream_t s);
  ~TimedLaunch();
  int id;
  hipStream_t stream;
  int slot;
};

}  // namespace fa
