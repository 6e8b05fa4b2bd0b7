// fa_api.hip -- the C ABI of libfa.so (declared in include/fa.h): argument
// validation, then kernel launches on the caller's stream.  Host-only code.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/fa.h"
#include "fa_launch.h"

// ---- fixed device scratch for fa_bwd_noalloc ----
// Holds the two float32 row arrays fa_bwd keeps in the caller's workspace.
// A file-scope device array: every GPU the library runs on holds one copy,
// allocated when the code object is loaded, until the process ends.  In host
// code `scratch` names a host-side stand-in, never the device copy: its
// device address is looked up once per device with hipGetSymbolAddress and
// only that address is handed to kernels.
constexpr size_t kScratchBytes = size_t(32) << 20;  // 32 MiB: B*H*N up to 2^22 rows
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxN = 1 << 23;  // one head's tensor stays below 4 GiB (buffer range)
constexpr double kMaxRows = 1073741824.0;  // B*H*N rows at most (2^30)
// Grids are padded per head: the largest is the 8-wave forward's
// B*H*ceil(N/256) workgroups of 512 work-items, at most
// B*H*ceil(N/64) * 512.  Keeping B*H*ceil(N/64) below 2^23 keeps every
// launch below 2^32 work-items (and every workgroup count an int).
constexpr double kMaxPaddedBlocks = 8388608.0;  // 2^23
constexpr long long kMaxPos = 1LL << 62;    // partial attention positions
constexpr float kMinScale = 0x1p-32f;        // accepted softmax scales
constexpr float kMaxScale = 0x1p32f;

bool aligned16(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shapes and scale; returns FA_OK or the status to report.
int check_problem(int dtype, int B, int H, int N, int D, float scale) {
  if (dtype != FA_F32 && dtype != FA_BF16 && dtype != FA_F16) return FA_ERR_UNSUPPORTED;
  if (B <= 0 || H <= 0 || N <= 0 || N > kMaxN) return FA_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
  if ((double)B * H * N > kMaxRows) return FA_ERR_INVALID_ARG;
  if ((double)B * H * ((N + 63) / 64) >= kMaxPaddedBlocks) return FA_ERR_INVALID_ARG;
  // scale * log2(e) is folded into one fp32 factor and divided back out of
  // the seeded accumulators: keep it a normal number with room either side.
  if (!(scale >= kMinScale && scale <= kMaxScale)) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

size_t delta_bytes(int B, int H, int N) {
  size_t n = (size_t)B * H * N * sizeof(float);
  return (n + 255) & ~(size_t)255;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, looked up on the first
// call on that device.  The caller's stream must belong to the current
// device (the lookup and the kernels must agree on the GPU).
int device_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return FA_ERR_HIP;
    if (sdev != dev) return FA_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

extern "C" int fa_version(void) { return 4; }

extern "C" const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported dtype or head dimension";
    case FA_ERR_WORKSPACE: return "workspace missing or too small";
    case FA_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

extern "C" int fa_fwd(int dtype, int B, int H, int N, int D, float scale, int causal,
                      const void* Q, const void* K, const void* V, void* O, float* LSE,
                      void* stream) {
  int rc = check_problem(dtype, B, H, N, D, scale);
  if (rc != FA_OK) return rc;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE))
    return FA_ERR_INVALID_ARG;
  fa::FwdArgs a{dtype, B, H, N, N, D, 0, scale, causal ? 1 : 0, Q, K, V, O, LSE,
                (hipStream_t)stream};
  hipError_t e;
  {
    fa::TimedLaunch t(FA_KERNEL_FWD, a.stream);
    e = fa::launch_fwd(a);
  }
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int fa_fwd_partial(int dtype, int B, int H, int Nq, int Nk, int D, float scale,
                              int causal, long long q_pos, long long k_pos, const void* Q,
                              const void* K, const void* V, void* O, float* LSE,
                              void* stream) {
  int rc = check_problem(dtype, B, H, Nq, D, scale);
  if (rc != FA_OK) return rc;
  rc = check_problem(dtype, B, H, Nk, D, scale);
  if (rc != FA_OK) return rc;
  if (q_pos < 0 || k_pos < 0 || q_pos > kMaxPos || k_pos > kMaxPos) return FA_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE))
    return FA_ERR_INVALID_ARG;
  // Key j is visible to query i iff k_pos + j <= q_pos + i, i.e. j <= i + d.
  // d >= Nk - 1 makes every key visible (the unmasked kernels); d <= -Nq
  // hides every key, and any such d behaves like -Nq.
  long long d = q_pos - k_pos;
  int mask = causal ? 1 : 0;
  if (mask && d >= (long long)Nk - 1) mask = 0;
  if (d < -(long long)Nq) d = -(long long)Nq;
  if (d > (long long)Nk) d = Nk;
  fa::FwdArgs a{dtype, B, H, Nq, Nk, D, (int)d, scale, mask, Q, K, V, O, LSE,
                (hipStream_t)stream};
  hipError_t e;
  {
    fa::TimedLaunch t(FA_KERNEL_FWD, a.stream);
    e = fa::launch_fwd(a);
  }
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int fa_merge(int dtype, int B, int H, int N, int D, void* O, float* LSE,
                        const void* O_part, const float* LSE_part, void* stream) {
  int rc = check_problem(dtype, B, H, N, D, 1.f);
  if (rc != FA_OK) return rc;
  if (!aligned16(O) || !aligned16(LSE) || !aligned16(O_part) || !aligned16(LSE_part))
    return FA_ERR_INVALID_ARG;
  fa::MergeArgs a{dtype, B, H, N, D, O, LSE, O_part, LSE_part, (hipStream_t)stream};
  hipError_t e;
  {
    fa::TimedLaunch t(FA_KERNEL_MERGE, a.stream);
    e = fa::launch_merge(a);
  }
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" size_t fa_bwd_workspace_bytes(int dtype, int B, int H, int N, int D, int causal) {
  (void)causal;
  if (dtype == FA_F32 || check_problem(dtype, B, H, N, D, 1.f) != FA_OK) return 0;
  return 2 * delta_bytes(B, H, N);
}

namespace {

// Validation shared by fa_bwd and fa_bwd_noalloc.
int check_bwd(int dtype, int B, int H, int N, int D, float scale, const void* Q, const void* K,
              const void* V, const void* O, const void* dO, const float* LSE, const void* dQ,
              const void* dK, const void* dV) {
  int rc = check_problem(dtype, B, H, N, D, scale);
  if (rc != FA_OK) return rc;
  if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;  // backward kernels are 16-bit only
  const void* ptrs[] = {Q, K, V, O, dO, LSE, dQ, dK, dV};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

// The three backward kernels on `a.stream`.
int launch_bwd(const fa::BwdArgs& a) {
  hipError_t e;
  {
    fa::TimedLaunch t(FA_KERNEL_BWD_DELTA, a.stream);
    e = fa::launch_bwd_delta(a);
  }
  if (e != hipSuccess) return FA_ERR_HIP;
  if (fa::bwd_combined(a)) {  // small D = 64 grids: dK/dV and dQ in one launch
    fa::TimedLaunch t(FA_KERNEL_BWD_DKDV_DQ, a.stream);
    e = fa::launch_bwd_dkdv_dq(a);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
  }
  {
    fa::TimedLaunch t(FA_KERNEL_BWD_DKDV, a.stream);
    e = fa::launch_bwd_dkdv(a);
  }
  if (e != hipSuccess) return FA_ERR_HIP;
  {
    fa::TimedLaunch t(FA_KERNEL_BWD_DQ, a.stream);
    e = fa::launch_bwd_dq(a);
  }
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" int fa_bwd(int dtype, int B, int H, int N, int D, float scale, int causal,
                      const void* Q, const void* K, const void* V, const void* O,
                      const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                      void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_bwd(dtype, B, H, N, D, scale, Q, K, V, O, dO, LSE, dQ, dK, dV);
  if (rc != FA_OK) return rc;
  const size_t rows_bytes = delta_bytes(B, H, N);
  if (!workspace || workspace_bytes < 2 * rows_bytes) return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_INVALID_ARG;
  float* ndelta = (float*)workspace;
  float* nlse = (float*)((char*)workspace + rows_bytes);
  fa::BwdArgs a{dtype, B, H, N, D, scale, causal ? 1 : 0, Q, K, V, O, dO, LSE,
                dQ, dK, dV, ndelta, nlse, (hipStream_t)stream};
  return launch_bwd(a);
}

extern "C" size_t fa_bwd_noalloc_max_bytes(void) { return kScratchBytes; }

extern "C" int fa_bwd_noalloc(int dtype, int B, int H, int N, int D, float scale, int causal,
                              const void* Q, const void* K, const void* V, const void* O,
                              const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                              void* stream) {
  int rc = check_bwd(dtype, B, H, N, D, scale, Q, K, V, O, dO, LSE, dQ, dK, dV);
  if (rc != FA_OK) return rc;
  const size_t rows_bytes = delta_bytes(B, H, N);
  if (2 * rows_bytes > kScratchBytes) return FA_ERR_WORKSPACE;
  void* base = nullptr;
  rc = device_scratch((hipStream_t)stream, &base);
  if (rc != FA_OK) return rc;
  // Every element the kernels read from the scratch is written first by the
  // Delta kernel of this same call, so nothing needs clearing.
  float* ndelta = (float*)base;
  float* nlse = (float*)((char*)base + rows_bytes);
  fa::BwdArgs a{dtype, B, H, N, D, scale, causal ? 1 : 0, Q, K, V, O, dO, LSE,
                dQ, dK, dV, ndelta, nlse, (hipStream_t)stream};
  return launch_bwd(a);
}
