// fa_bwd.hip -- backward kernels with on-chip recomputation of S and P.
//
// Pages cited (by address and title):
//   [csdn]      adg.csdn.net/6a311d0d10ee7a33f27dee1b.html
//               "kk的大模型论文学习笔记 第8篇: FlashAttention"
//   [guanweilu] guanweilu.cn/article/445.html
//               "CUDA Kernel 级别的优化：Flash Attention 为什么比 PyTorch 原生实现快 5-10 倍"
//
// The pages' backward pass keeps no N x N matrix: it recomputes S and P on
// chip when the gradients need them, because recomputing is cheaper than a
// round trip through HBM ([csdn] "重计算：扔掉比存着更快"; [guanweilu]
// "FlashAttention 的三板斧", third technique).  P is rebuilt from the saved
// per-row log-sum-exp: P_ij = exp(scale q_i.k_j - LSE_i).
//
// Gradients of sum(O * dO) (plain calculus of O = softmax(scale Q K^T) V):
//   dV = P^T dO,  dP = dO V^T,  Delta_i = sum_j P_ij dP_ij = dO_i . O_i,
//   dS = P * (dP - Delta),  dQ = scale dS K,  dK = scale dS^T Q.
//
// Three kernels, no atomics (bit-for-bit repeatable):
//   1. delta: -Delta_i = -dO_i . O_i and -LSE_i / scale, float32, into the
//             caller's workspace (negated so they can seed accumulators).
//   2. dkdv:  a workgroup keeps 128 key rows resident (each wave 32 keys, K and
//             V as VGPR operands, dK^T and dV^T accumulators in VGPRs) and
//             streams query tiles (Q, dO, LSE, Delta) into double-buffered LDS
//             with direct global->LDS loads.  Per 32x32 block: S = Q K^T and
//             dP = dO V^T leave one key per lane, so P and dS feed straight in
//             as B operands of dV^T += dO^T P and dK^T += Q^T dS, whose A
//             operands come from the same row-major Q and dO tiles through
//             transposing LDS reads.  The S and dP accumulators start at
//             -LSE/scale and -Delta of their query rows instead of zero, so
//             the MFMAs leave S - LSE/scale and dP - Delta: P is one multiply
//             and an exp2, dS one multiply.
//   3. dq:    a workgroup keeps 128 query rows resident (Q, dO as operands,
//             LSE and Delta one scalar per lane) and streams key tiles (K, V).
//             S^T = K Q^T and dP^T = V dO^T leave one query per lane, so dS^T
//             feeds dQ^T += K^T dS^T directly (K^T by transposing reads).
//             Its S and dP accumulators start from register blocks holding
//             the lane's -LSE/scale and -Delta (an MFMA's C and D operands
//             may differ, so the seeds survive every tile).
// The dq kernel recomputes S and dP a second time; that costs two extra
// contractions per tile but removes every cross-workgroup reduction.
// At D = 64 the two need the same registers and LDS, and on grids of at most
// 8 workgroups per CU (e.g. B=8 H=12 N=1024, or one head group at N <= 8192)
// they run as one launch (bwd_dkdv_dq_kernel): one kernel boundary fewer,
// and dQ workgroups fill the CUs that the short causal dK/dV workgroups leave
// idle (measured -5 to -24%; on larger grids the shared launch was 2-5%
// slower, so those keep two launches).
#include <hip/hip_runtime.h>

#include <math.h>

#include <type_traits>

#include "fa_bwd_dkdv.h"
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

// ------------------------------------------------------------------ delta

// -Delta_i = -dO_i . O_i (fp32) and -LSE_i / scale, one row per D/8 lanes.
template <typename T, int D>
__global__ void __launch_bounds__(256)
bwd_delta_kernel(const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
                 const float* __restrict__ LSE, float* __restrict__ ndelta,
                 float* __restrict__ nlse, float inv_scale, size_t rows) {
  constexpr int TPR = D / 8;  // threads per row, 16 bytes each
  constexpr int RPB = 256 / TPR;
  const int part = threadIdx.x % TPR;
  // Grid-stride over rows; every lane of a wave runs the same number of
  // iterations (the bound is per workgroup), so the shuffles stay converged.
  for (size_t row0 = (size_t)blockIdx.x * RPB; row0 < rows; row0 += (size_t)gridDim.x * RPB) {
    const size_t row = row0 + threadIdx.x / TPR;
    float acc = 0.f;
    if (row < rows) {
      const u32x4 o = ld_global16(O + row * D + part * 8);
      const u32x4 g = ld_global16(dO + row * D + part * 8);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc = fmaf(T::to_float(elem16(o, j)), T::to_float(elem16(g, j)), acc);
    }
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (row < rows && part == 0) {
      ndelta[row] = -acc;
      nlse[row] = -LSE[row] * inv_scale;
    }
  }
}

// ------------------------------------------------------------------ dQ

template <int D>
struct DqTile;
template <>
struct DqTile<64> {
  static constexpr int BC = 64;  // key rows per streamed tile
};
template <>
struct DqTile<128> {
  static constexpr int BC = 32;
};

constexpr int kDqBR = 128;  // query rows per workgroup (4 waves x 32)

template <int D>
constexpr int dq_stage_elems() { return 2 * DqTile<D>::BC * D; }

// The dQ work of workgroup `pid` (the query-resident kernel described at
// the top of this file), on two LDS stages of dq_stage_elems<D>() elements
// each.  Shared by bwd_dq_kernel and the combined launch below.
template <typename T, int D, bool CAUSAL>
__device__ __forceinline__ void dq_body(const uint16_t* __restrict__ Q,
                                        const uint16_t* __restrict__ K,
                                        const uint16_t* __restrict__ V,
                                        const uint16_t* __restrict__ dO,
                                        const float* __restrict__ nlse,
                                        const float* __restrict__ ndelta,
                                        uint16_t* __restrict__ dQ, int N, float c, float scale,
                                        int nqt, int total, int tile_major, int pid,
                                        uint16_t* smem0, uint16_t* smem1) {
  constexpr int BC = DqTile<D>::BC;
  constexpr int TILE = BC * D;             // elements of one K or V tile
  constexpr int BLOCKS = TILE * 2 / 1024;  // 1 KiB blocks per tile
  constexpr int NKB = BC / 32;
  constexpr int NDC = D / 16;
  constexpr int NDB = D / 32;
  constexpr int NKC = BC / 16;
  static_assert(BLOCKS == 8, "two blocks of K and two of V per wave");


  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int l32 = lane & 31, hh = lane >> 5;

  int bh, qt;
  tile_of(pid, total, nqt, tile_major, bh, qt);
  if (CAUSAL) qt = nqt - 1 - qt;  // longest rows first
  const int q0 = qt * kDqBR;
  const int wq0 = q0 + wave * 32;
  const int myq = wq0 + l32;

  const size_t base = (size_t)bh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const auto rQ = make_rsrc(Q + base, head_bytes);
  const auto rdO = make_rsrc(dO + base, head_bytes);
  const i32x4 rK = rsrc_words(K + base, head_bytes);  // direct-to-LDS sources
  const i32x4 rV = rsrc_words(V + base, head_bytes);

  const int kend = CAUSAL ? min(N, q0 + kDqBR) : N;
  const int ntiles = (kend + BC - 1) / BC;

  auto dma = [&](const uint16_t* S0, int ts) {
#pragma unroll
    for (int i = 0; i < BLOCKS / 4; ++i) {
      const int b = wave_u + 4 * i;
      const uint32_t goff = dma_goff<D>(b, lane, ts);
      lds_dma16(rK, S0 + b * 512, goff);
      lds_dma16(rV, S0 + TILE + b * 512, goff);
    }
  };

  const int nfull = min(N / BC, CAUSAL ? (q0 + 1) / BC : ntiles);
  // The first key tile travels while Q and dO load.
  if (ntiles > 0) dma(smem0, 0);

  u32x4 qf[NDC], gf[NDC];
#pragma unroll
  for (int cc = 0; cc < NDC; ++cc) {
    const uint32_t off = ((uint32_t)myq * D + 16 * cc + 8 * hh) * 2u;
    qf[cc] = buf_load16(rQ, off);
    gf[cc] = buf_load16(rdO, off);
  }
#pragma unroll
  for (int cc = 0; cc < NDC; ++cc) {
    settle(qf[cc]);
    settle(gf[cc]);
  }
  const auto rL = make_rsrc(nlse + (size_t)bh * N, (uint32_t)N * 4);
  const auto rD = make_rsrc(ndelta + (size_t)bh * N, (uint32_t)N * 4);
  // Seeds of the S and dP accumulators: every register of a lane holds the
  // lane's query, so S starts at -LSE/scale and dP at -Delta in all 16.
  const float nls = buf_load_f32(rL, (uint32_t)myq * 4u);
  const float ndlt = buf_load_f32(rD, (uint32_t)myq * 4u);  // -Delta
  settle(nls);
  settle(ndlt);
  f32x16 seed_s, seed_dp;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    seed_s[r] = nls;
    seed_dp[r] = ndlt;
  }

  int roff[NDC];
#pragma unroll
  for (int cc = 0; cc < NDC; ++cc) roff[cc] = toff<D>(l32, 16 * cc + 8 * hh);
  const int G = lane >> 4, a16 = lane & 15;
  int toffs[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int t = 0; t < 2; ++t)
      toffs[db][t] = toff<D>(8 * t + 4 * (G >> 1) + (a16 >> 2), 32 * db + 16 * (G & 1) + 4 * (a16 & 3));

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

  // One key tile.  MASKED: a ragged tail or a tile on the causal diagonal of
  // this workgroup's rows (per-wave skip, element mask); otherwise the body
  // is straight-line code.
  auto tile = [&](const uint16_t* S0, int ts, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    const uint16_t* Ks = S0;
    const uint16_t* Vs = S0 + TILE;
    if (MASKED && CAUSAL && ts > wq0 + 31) return;  // no key visible to this wave
    const bool need_mask = MASKED && ((ts + BC > N) || (CAUSAL && ts + BC - 1 > wq0));
    f32x16 s[NKB], dp[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      s[kb] = seed_s;
      dp[kb] = seed_dp;
    }
#pragma unroll
    for (int cc = 0; cc < NDC; ++cc)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[kb] = T::mfma(ld_lds16(Ks + kb * 32 * D + roff[cc]), qf[cc], s[kb]);
        dp[kb] = T::mfma(ld_lds16(Vs + kb * 32 * D + roff[cc]), gf[cc], dp[kb]);
      }
    // lane: query `myq`; register r of block kb: key ts + kb*32 + 8*(r/4) + 4*hh + r%4
    u32x4 dsk[NKC];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float ds2[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int r = 8 * half + 2 * i + e;
            float pv = fast_exp2(s[kb][r] * c);
            if (need_mask) {
              const int key = ts + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
              if (key >= N || (CAUSAL && key > myq)) pv = 0.f;
            }
            ds2[e] = pv * dp[kb][r];
          }
          dsk[2 * kb + half][i] = T::pack2(ds2[0], ds2[1]);
        }
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const uint16_t* kb16 = Ks + kc * 16 * D;
        const u32x4 a = cat(ld_lds_tr(kb16 + toffs[db][0]), ld_lds_tr(kb16 + toffs[db][1]));
        acc[db] = T::mfma(a, dsk[kc], acc[db]);
      }
    // two accumulator chains: keep the K^T reads three MFMAs ahead
    if constexpr (!MASKED) pipeline_reads<NKC * NDB, 2, 3, 1>();
  };

  // Tiles wholly visible to every row of the workgroup (no tail, not past
  // the causal diagonal) come first and run the straight-line body; the rest
  // (at the end) run the masked body.  All of them are double-buffered: tile
  // t sits in stage t % 2 and the next one loads while it is consumed.
  int t = 0;
  wait_dma();
  __syncthreads();
  for (; t < nfull; t += 2) {
    if (t + 1 < ntiles) dma(smem1, (t + 1) * BC);
    tile(smem0, t * BC, std::false_type());
    wait_dma();
    __syncthreads();
    if (t + 1 >= nfull) {
      t += 1;
      break;
    }
    if (t + 2 < ntiles) dma(smem0, (t + 2) * BC);
    tile(smem1, (t + 1) * BC, std::false_type());
    wait_dma();
    __syncthreads();
  }
  // One copy of the masked body, its stage picked at run time (a copy per
  // stage made the compiler spill registers at D = 128).
  for (; t < ntiles; ++t) {
    const bool odd = t & 1;
    if (t + 1 < ntiles) dma(odd ? smem0 : smem1, (t + 1) * BC);
    tile(odd ? smem1 : smem0, t * BC, std::true_type());
    wait_dma();
    __syncthreads();
  }

  if (myq < N) {
    uint16_t* dQr = dQ + base + (size_t)myq * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = T::pack2(acc[db][4 * g] * scale, acc[db][4 * g + 1] * scale);
        w[1] = T::pack2(acc[db][4 * g + 2] * scale, acc[db][4 * g + 3] * scale);
        st_global8(dQr + db * 32 + 8 * g + 4 * hh, w);
      }
  }
}

template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(256, 2)
bwd_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
              const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
              const float* __restrict__ nlse, const float* __restrict__ ndelta,
              uint16_t* __restrict__ dQ, int N, float c, float scale, int nqt, int total,
              int tile_major) {
  __shared__ __attribute__((aligned(1024))) uint16_t smem0[dq_stage_elems<D>()];
  __shared__ __attribute__((aligned(1024))) uint16_t smem1[dq_stage_elems<D>()];
  dq_body<T, D, CAUSAL>(Q, K, V, dO, nlse, ndelta, dQ, N, c, scale, nqt, total, tile_major,
                        blockIdx.x, smem0, smem1);
}

// D = 64: the dK/dV and dQ workgroups of one backward in a single launch.
// Both need the same registers and LDS and neither reads the other's output,
// so sharing a grid removes a kernel boundary and lets one kernel's short
// tail tiles fill in beside the other's.  Roles alternate every 8 workgroups
// (one per XCD), so each XCD gets the same mix and, within a role, workgroup
// `pid` keeps pid % 8 == its XCD as the tile order assumes.
template <typename T, bool CAUSAL>
__global__ void __launch_bounds__(256, 2)
bwd_dkdv_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                   const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                   const float* __restrict__ nlse, const float* __restrict__ ndelta,
                   uint16_t* __restrict__ dQ, uint16_t* __restrict__ dK,
                   uint16_t* __restrict__ dV, int N, float c, float scale, int nkt, int total_kv,
                   int tm_kv, int nqt, int total_q, int tm_q) {
  constexpr int D = 64;
  constexpr int E = dkv_stage_elems<D>() > dq_stage_elems<D>() ? dkv_stage_elems<D>()
                                                               : dq_stage_elems<D>();
  __shared__ __attribute__((aligned(1024))) uint16_t smem0[E];
  __shared__ __attribute__((aligned(1024))) uint16_t smem1[E];
  const int b = blockIdx.x;
  const int pid = ((b >> 4) << 3) | (b & 7);
  if (((b >> 3) & 1) == 0) {
    if (pid < total_kv)
      dkdv_body<T, D, CAUSAL>(Q, K, V, dO, nlse, ndelta, dK, dV, N, c, scale, nkt, total_kv,
                              tm_kv, pid, smem0, smem1);
  } else {
    if (pid < total_q)
      dq_body<T, D, CAUSAL>(Q, K, V, dO, nlse, ndelta, dQ, N, c, scale, nqt, total_q, tm_q, pid,
                            smem0, smem1);
  }
}

template <typename T, bool CAUSAL>
static hipError_t dkdv_dq64(const BwdArgs& a) {
  const int nkt = (a.N + kDkvKeys - 1) / kDkvKeys;
  const int total_kv = nkt * a.B * a.H;
  const int nqt = (a.N + kDqBR - 1) / kDqBR;
  const int total_q = nqt * a.B * a.H;
  const int mx = total_kv > total_q ? total_kv : total_q;
  const unsigned grid = 16u * (unsigned)((mx + 7) / 8);
  hipLaunchKernelGGL((bwd_dkdv_dq_kernel<T, CAUSAL>), dim3(grid), dim3(256), 0, a.stream,
                     (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V,
                     (const uint16_t*)a.dO, a.nlse, a.ndelta, (uint16_t*)a.dQ, (uint16_t*)a.dK,
                     (uint16_t*)a.dV, a.N, a.scale * kLog2e, a.scale, nkt, total_kv,
                     tile_major(CAUSAL, nkt, total_kv), nqt, total_q,
                     tile_major(CAUSAL, nqt, total_q));
  return hipGetLastError();
}

bool bwd_combined(const BwdArgs& a) {
  if (a.D != 64) return false;
  const long n = (long)((a.N + kDqBR - 1) / kDqBR) * a.B * a.H;
  return 2 * n <= 8L * cu_count();  // grids of at most a few rounds
}

hipError_t launch_bwd_dkdv_dq(const BwdArgs& a) {
  if (a.dtype == kBF16) return a.causal ? dkdv_dq64<BF16, true>(a) : dkdv_dq64<BF16, false>(a);
  return a.causal ? dkdv_dq64<F16, true>(a) : dkdv_dq64<F16, false>(a);
}

// ------------------------------------------------------------------ launchers

template <typename T>
static hipError_t delta16(const BwdArgs& a) {
  const size_t rows = (size_t)a.B * a.H * a.N;
  const int rpb = 256 / (a.D / 8);
  const size_t blocks = (rows + rpb - 1) / rpb;
  const unsigned grid = (unsigned)(blocks < (1u << 20) ? blocks : (1u << 20));
  if (a.D == 64)
    hipLaunchKernelGGL((bwd_delta_kernel<T, 64>), dim3(grid), dim3(256), 0, a.stream,
                       (const uint16_t*)a.O, (const uint16_t*)a.dO, a.LSE, a.ndelta, a.nlse,
                       1.f / a.scale, rows);
  else
    hipLaunchKernelGGL((bwd_delta_kernel<T, 128>), dim3(grid), dim3(256), 0, a.stream,
                       (const uint16_t*)a.O, (const uint16_t*)a.dO, a.LSE, a.ndelta, a.nlse,
                       1.f / a.scale, rows);
  return hipGetLastError();
}

hipError_t launch_bwd_delta(const BwdArgs& a) {
  return a.dtype == kBF16 ? delta16<BF16>(a) : delta16<F16>(a);
}


template <typename T>
static hipError_t dkdv16(const BwdArgs& a) {
  if (a.D == 64) return a.causal ? dkdv<T, 64, true>(a) : dkdv<T, 64, false>(a);
  if (!a.causal) return launch_bwd_dkdv_d128_nomask(a);  // fa_bwd_d128.hip
  return dkdv<T, 128, true>(a);
}

hipError_t launch_bwd_dkdv(const BwdArgs& a) {
  return a.dtype == kBF16 ? dkdv16<BF16>(a) : dkdv16<F16>(a);
}

template <typename T, int D, bool CAUSAL>
static hipError_t dq(const BwdArgs& a) {
  const int nqt = (a.N + kDqBR - 1) / kDqBR;
  const int total = nqt * a.B * a.H;
  hipLaunchKernelGGL((bwd_dq_kernel<T, D, CAUSAL>), dim3(total), dim3(256), 0, a.stream,
                     (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V,
                     (const uint16_t*)a.dO, a.nlse, a.ndelta, (uint16_t*)a.dQ, a.N,
                     a.scale * kLog2e, a.scale, nqt, total, tile_major(CAUSAL, nqt, total));
  return hipGetLastError();
}

template <typename T>
static hipError_t dq16(const BwdArgs& a) {
  if (a.D == 64) return a.causal ? dq<T, 64, true>(a) : dq<T, 64, false>(a);
  return a.causal ? dq<T, 128, true>(a) : dq<T, 128, false>(a);
}

hipError_t launch_bwd_dq(const BwdArgs& a) {
  return a.dtype == kBF16 ? dq16<BF16>(a) : dq16<F16>(a);
}

}  // namespace fa
