// fa_merge.hip -- exact merge of two partial attention results.
//
// Page cited: [guanweilu] guanweilu.cn/article/445.html
//   "CUDA Kernel 级别的优化：Flash Attention 为什么比 PyTorch 原生实现快 5-10 倍",
//   "FlashAttention 的三板斧", second technique (online softmax).
//
// The online softmax carries (max, sum) per row from one key tile to the
// next; (O, LSE) of a finished pass over a key block carries the same
// information in closed form, since LSE = m + ln(l) and O is normalised.
// Two passes over disjoint key blocks therefore combine exactly:
//   LSE = ln(e^LSE_a + e^LSE_b),  O = e^(LSE_a - LSE) O_a + e^(LSE_b - LSE) O_b.
// A partial whose row saw no key (LSE = -inf) is the identity; two such
// partials merge to O = 0, LSE = -inf.
//
// The kernel is a pure stream over HBM: each thread owns 16 bytes of one row
// of O (8 bf16/f16 or 4 fp32 elements) and its two LSE values; rows are
// split over D/8 (or D/4) consecutive lanes so every wave reads and writes
// whole contiguous rows.  Grid-stride over rows keeps the grid bounded.
#include <hip/hip_runtime.h>

#include <math.h>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

// Weights of the two partials and the merged LSE for one row.
__device__ inline void merge_weights(float la, float lb, float& wa, float& wb, float& lse) {
  const float m = fmaxf(la, lb);
  if (m == -INFINITY) {  // neither partial saw a key
    wa = wb = 0.f;
    lse = -INFINITY;
    return;
  }
  const float ea = expf(la - m), eb = expf(lb - m);  // one of them is 1
  const float s = ea + eb;
  wa = ea / s;
  wb = eb / s;
  lse = m + logf(s);
}

}  // namespace

template <typename T, int D>
__global__ void __launch_bounds__(256)
merge16_kernel(uint16_t* O, float* LSE, const uint16_t* Ob, const float* LSEb, size_t rows) {
  constexpr int TPR = D / 8;  // threads per row
  constexpr int RPB = 256 / TPR;
  const int part = threadIdx.x % TPR;
  for (size_t row = (size_t)blockIdx.x * RPB + threadIdx.x / TPR; row < rows;
       row += (size_t)gridDim.x * RPB) {
    const float la = LSE[row], lb = LSEb[row];
    float wa, wb, lse;
    merge_weights(la, lb, wa, wb, lse);
    uint16_t* po = O + row * D + part * 8;
    const u32x4 a = ld_global16(po);
    const u32x4 b = ld_global16(Ob + row * D + part * 8);
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = wa * T::to_float(elem16(a, 2 * j)) + wb * T::to_float(elem16(b, 2 * j));
      const float hi =
          wa * T::to_float(elem16(a, 2 * j + 1)) + wb * T::to_float(elem16(b, 2 * j + 1));
      r[j] = T::pack2(lo, hi);
    }
    *reinterpret_cast<u32x4*>(po) = r;
    // The row's lanes sit in one wave and the new LSE depends on the loaded
    // one, so every lane's read has returned before part 0 overwrites it.
    if (part == 0) LSE[row] = lse;
  }
}

template <int D>
__global__ void __launch_bounds__(256)
merge32_kernel(float* O, float* LSE, const float* Ob, const float* LSEb, size_t rows) {
  constexpr int TPR = D / 4;
  constexpr int RPB = 256 / TPR;
  const int part = threadIdx.x % TPR;
  for (size_t row = (size_t)blockIdx.x * RPB + threadIdx.x / TPR; row < rows;
       row += (size_t)gridDim.x * RPB) {
    const float la = LSE[row], lb = LSEb[row];
    float wa, wb, lse;
    merge_weights(la, lb, wa, wb, lse);
    float* po = O + row * D + part * 4;
    const f32x4 a = *reinterpret_cast<const f32x4*>(po);
    const f32x4 b = *reinterpret_cast<const f32x4*>(Ob + row * D + part * 4);
    f32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = wa * a[j] + wb * b[j];
    *reinterpret_cast<f32x4*>(po) = r;
    if (part == 0) LSE[row] = lse;
  }
}

namespace {

constexpr unsigned kMaxMergeGrid = 1u << 16;  // workgroups; rows beyond loop

unsigned merge_grid(size_t rows, int rpb) {
  const size_t g = (rows + rpb - 1) / rpb;
  return (unsigned)(g < kMaxMergeGrid ? g : kMaxMergeGrid);
}

template <typename T>
hipError_t merge16(const MergeArgs& a) {
  const size_t rows = (size_t)a.B * a.H * a.N;
  const unsigned grid = merge_grid(rows, 256 / (a.D / 8));
  if (a.D == 64)
    hipLaunchKernelGGL((merge16_kernel<T, 64>), dim3(grid), dim3(256), 0, a.stream,
                       (uint16_t*)a.O, a.LSE, (const uint16_t*)a.Ob, a.LSEb, rows);
  else
    hipLaunchKernelGGL((merge16_kernel<T, 128>), dim3(grid), dim3(256), 0, a.stream,
                       (uint16_t*)a.O, a.LSE, (const uint16_t*)a.Ob, a.LSEb, rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a) {
  if (a.dtype == kBF16) return merge16<BF16>(a);
  if (a.dtype == kF16) return merge16<F16>(a);
  const size_t rows = (size_t)a.B * a.H * a.N;
  const unsigned grid = merge_grid(rows, 256 / (a.D / 4));
  if (a.D == 64)
    hipLaunchKernelGGL((merge32_kernel<64>), dim3(grid), dim3(256), 0, a.stream, (float*)a.O,
                       a.LSE, (const float*)a.Ob, a.LSEb, rows);
  else
    hipLaunchKernelGGL((merge32_kernel<128>), dim3(grid), dim3(256), 0, a.stream, (float*)a.O,
                       a.LSE, (const float*)a.Ob, a.LSEb, rows);
  return hipGetLastError();
}

}  // namespace fa
