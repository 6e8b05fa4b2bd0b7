// fa_probe.hip -- measurement probe, built as its own library (libfa_probe.so),
// not part of the attention ABI.
//
// Rate of fp32 updates to device memory, the operation a backward pass that
// accumulated dQ across key blocks in global memory would be built on:
// plain stores, plain read-modify-write, and fp32 atomic adds (relaxed,
// device scope, result unused, so the hardware's global_atomic_add_f32).
// Every element of the buffer is updated once per pass by exactly one lane
// (a grid-stride loop, 256 consecutive bytes per wave), so the atomic rate
// measured is the uncontended one: an upper bound for that design.
#include <hip/hip_runtime.h>

#include <stddef.h>

namespace {

template <int MODE>  // 0: store 1.0f, 1: x += 1.0f, 2: atomic x += 1.0f
__global__ void __launch_bounds__(256) update_kernel(float* __restrict__ buf, size_t n,
                                                      int passes) {
  const size_t stride = (size_t)gridDim.x * 256;
  for (int p = 0; p < passes; ++p)
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
      if constexpr (MODE == 0)
        buf[i] = 1.0f;
      else if constexpr (MODE == 1)
        buf[i] += 1.0f;
      else
        __hip_atomic_fetch_add(buf + i, 1.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace

// Launches `passes` update passes over buf[0, n) on `stream`: mode 0 plain
// stores, 1 plain read-modify-write, 2 fp32 atomic adds.  Returns 0, or a
// hipError_t value (invalid mode or size: hipErrorInvalidValue).  The grid
// is 8 workgroups of 256 lanes per compute unit, so the launch does not
// depend on n beyond the loop count.
extern "C" int fa_probe_update(int mode, float* buf, size_t n, int passes, hipStream_t stream) {
  if (buf == nullptr || n == 0 || passes < 1 || mode < 0 || mode > 2)
    return (int)hipErrorInvalidValue;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return (int)e;
  size_t blocks = (size_t)(cus > 0 ? cus : 256) * 8;
  const size_t need = (n + 255) / 256;
  if (blocks > need) blocks = need;
  const dim3 grid((unsigned)blocks), block(256);
  if (mode == 0)
    hipLaunchKernelGGL(update_kernel<0>, grid, block, 0, stream, buf, n, passes);
  else if (mode == 1)
    hipLaunchKernelGGL(update_kernel<1>, grid, block, 0, stream, buf, n, passes);
  else
    hipLaunchKernelGGL(update_kernel<2>, grid, block, 0, stream, buf, n, passes);
  return (int)hipGetLastError();
}
