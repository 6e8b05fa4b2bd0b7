// fa_bwd_d128.hip -- the dK/dV kernel for D = 128 without a mask, in a unit
// of its own so that it can be compiled with MFMA results kept in VGPRs
// (the build passes -mllvm -amdgpu-mfma-vgpr-form for this file only).
//
// At D = 128 the kernel holds K, V (64 registers), the dK^T, dV^T
// accumulators (128) and a tile's S, dP (32) per lane: more than 256, so it
// runs one wave per SIMD with AGPRs.  Left to its default, the compiler put
// the dK/dV accumulators in AGPRs but moved them through VGPRs around every
// tile (about 350 register moves per 32 MFMAs); with VGPR-form MFMAs and one
// tile per loop iteration it keeps them in place (no moves; measured 7.94 ->
// 6.24 ms for the whole backward at B=1, H=16, N=16384).  The masked variant
// and the D = 64 kernels measured no better this way and stay in fa_bwd.hip.
#include "fa_bwd_dkdv.h"
#include "fa_launch.h"

namespace fa {

hipError_t launch_bwd_dkdv_d128_nomask(const BwdArgs& a) {
  return a.dtype == kBF16 ? dkdv<BF16, 128, false>(a) : dkdv<F16, 128, false>(a);
}

}  // namespace fa
