/*
 * fa_probe.h -- C ABI of libfa_probe.so, measurement probes built beside
 * libfa.so.  Not part of the attention ABI: the callers are measurement
 * tools (bench.py --probe) that need the chip's own rates to read the
 * attention kernels' results against.
 *
 * Both entry points take a DEVICE pointer owned by the caller, enqueue one
 * kernel on `stream` (a hipStream_t; NULL = the null stream) and return.
 * Return value: 0, hipErrorInvalidValue (1) for bad arguments (checked
 * before any HIP call; nothing is launched), or the hipError_t of the
 * launch.
 */
#ifndef FA_PROBE_H
#define FA_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Updates every float of buf[0, n) `passes` times: mode 0 stores 1.0f,
 * mode 1 adds 1.0f with a plain load and store, mode 2 adds 1.0f with a
 * relaxed device-scope fp32 atomic (result unused).  One lane per element
 * per pass, 256 contiguous bytes per wave (no two lanes on one address).
 * Requires mode in {0, 1, 2}, buf != NULL, n >= 1, passes >= 1. */
int fa_probe_update(int mode, float* buf, size_t n, int passes, void* stream);

/* `blocks` workgroups of 4 waves; each wave runs 4 x `iters` dense bf16
 * MFMAs (32x32x16, four independent chains, register operands only) and
 * writes one float per lane to out[0, blocks * 256), which the caller
 * provides.  Requires out != NULL, blocks >= 1, iters >= 1. */
int fa_probe_mfma(float* out, int blocks, int iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_PROBE_H */
