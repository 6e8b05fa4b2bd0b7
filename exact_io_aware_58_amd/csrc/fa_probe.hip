// fa_probe.hip -- measurement probes, built as their own library
// (libfa_probe.so), not part of the attention ABI.
//
// fa_probe_mfma: the dense bf16 MFMA rate the chip sustains with register
// operands only, i.e. the matrix-core ceiling at the clock it holds.
//
// fa_probe_update: rate of fp32 updates to device memory, the operation a backward pass that
// accumulated dQ across key blocks in global memory would be built on:
// plain stores, plain read-modify-write, and fp32 atomic adds (relaxed,
// device scope, result unused, so the hardware's global_atomic_add_f32).
// Every element of the buffer is updated once per pass by exactly one lane
// (a grid-stride loop, 256 consecutive bytes per wave), so the atomic rate
// measured is the uncontended one: an upper bound for that design.
#include <hip/hip_runtime.h>

#include <stddef.h>

#include "../../include/fa_probe.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Dense bf16 MFMA rate with register operands only: every wave runs `iters`
// rounds of four independent 32x32x16 MFMA chains (no memory traffic in the
// loop), then stores one float per lane so that nothing is dropped.
__global__ void __launch_bounds__(256) mfma_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(lane + i));
    b[i] = (__bf16)(0.002f * (float)(lane - i));
  }
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  float sum = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) sum += c0[r] + c1[r] + c2[r] + c3[r];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = sum;
}

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
extern "C" int fa_probe_update(int mode, float* buf, size_t n, int passes, void* stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
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

// Launches the register-only MFMA probe: `blocks` workgroups of 4 waves, each
// wave 4 x `iters` dense bf16 MFMAs of 32x32x16 (32768 flops each).  `out`
// holds blocks x 256 floats (one per lane).  Returns 0 or a hipError_t value
// (bad arguments: hipErrorInvalidValue, before any HIP call).
extern "C" int fa_probe_mfma(float* out, int blocks, int iters, void* stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (out == nullptr || blocks < 1 || iters < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_kernel, dim3(blocks), dim3(256), 0, stream, out, iters);
  return (int)hipGetLastError();
}
