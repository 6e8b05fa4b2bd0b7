// fa_bwd_dkdv.h -- the key-resident dK/dV kernel of the backward pass
// (included by fa_bwd.hip and fa_bwd_d128.hip; see fa_bwd.hip for the
// method and the page citations).
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

// ------------------------------------------------------------------ dK, dV

template <int D>
struct DkvTile;
template <>
struct DkvTile<64> {
  static constexpr int BR = 64;     // query rows per streamed tile
  static constexpr int MIN_WG = 2;  // workgroups per CU the registers must allow
};
template <>
struct DkvTile<128> {
  static constexpr int BR = 32;
  static constexpr int MIN_WG = 1;  // K, V, dK, dV of 32 rows x 128 need > 256 VGPRs
};

constexpr int kDkvKeys = 128;  // key rows per workgroup (4 waves x 32)

// LDS elements of one dK/dV stage: Q, dO, then 64 -LSE/scale + 64 -Delta floats.
template <int D>
constexpr int dkv_stage_elems() { return 2 * DkvTile<D>::BR * D + 2 * 64 * 2; }

// The dK/dV work of workgroup `pid` (the key-resident kernel described at
// the top of fa_bwd.hip), on two LDS stages of dkv_stage_elems<D>()
// elements each.  Shared by bwd_dkdv_kernel and, at D = 64, the combined
// dK/dV + dQ launch (fa_bwd.hip).
template <typename T, int D, bool CAUSAL>
__device__ __forceinline__ void dkdv_body(const uint16_t* __restrict__ Q,
                                          const uint16_t* __restrict__ K,
                                          const uint16_t* __restrict__ V,
                                          const uint16_t* __restrict__ dO,
                                          const float* __restrict__ nlse,
                                          const float* __restrict__ ndelta,
                                          uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
                                          int N, float c, float scale, int nkt, int total,
                                          int tile_major, int pid, uint16_t* smem0,
                                          uint16_t* smem1) {
  constexpr int BR = DkvTile<D>::BR;
  constexpr int TILE = BR * D;                  // elements of one Q or dO tile
  constexpr int BLOCKS = TILE * 2 / 1024;       // 1 KiB blocks per tile
  constexpr int NDC = D / 16;
  constexpr int NDB = D / 32;
  static_assert(BLOCKS == 8, "two blocks of Q and two of dO per wave");

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int l32 = lane & 31, hh = lane >> 5;

  int bh, kt;  // causal: small kt has the most queries, runs first
  tile_of(pid, total, nkt, tile_major, bh, kt);
  const int k0 = kt * kDkvKeys;
  const int wk0 = k0 + wave_u * 32;
  const int mykey = wk0 + l32;

  const size_t base = (size_t)bh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const i32x4 rQ = rsrc_words(Q + base, head_bytes);  // direct-to-LDS sources
  const i32x4 rdO = rsrc_words(dO + base, head_bytes);
  const i32x4 rL = rsrc_words(nlse + (size_t)bh * N, (uint32_t)N * 4);
  const i32x4 rD = rsrc_words(ndelta + (size_t)bh * N, (uint32_t)N * 4);
  const auto rK = make_rsrc(K + base, head_bytes);
  const auto rV = make_rsrc(V + base, head_bytes);

  const int qstart = CAUSAL ? k0 : 0;  // earlier queries see none of these keys
  const int ntiles = qstart < N ? (N - qstart + BR - 1) / BR : 0;

  // Direct global->LDS loads of one query tile: each wave two blocks of Q and
  // two of dO; wave 0 also 64 -LSE/scale values, wave 1 64 -Delta values.
  // Rows past N arrive as zeros (then P = 1 but dO = Q = 0: no contribution).
  auto dma = [&](const uint16_t* S0, int qs) {
#pragma unroll
    for (int i = 0; i < BLOCKS / 4; ++i) {
      const int b = wave_u + 4 * i;
      const uint32_t goff = dma_goff<D>(b, lane, qs);
      lds_dma16(rQ, S0 + b * 512, goff);
      lds_dma16(rdO, S0 + TILE + b * 512, goff);
    }
    if (wave_u == 0)
      lds_dma4(rL, S0 + 2 * TILE, (uint32_t)(qs + lane) * 4u);
    else if (wave_u == 1)
      lds_dma4(rD, S0 + 2 * TILE + 128, (uint32_t)(qs + lane) * 4u);
  };

  // The first query tile travels while K and V load.
  if (ntiles > 0) dma(smem0, qstart);

  // B operands of S = Q K^T and dP = dO V^T: lane holds row `mykey` of K, V.
  u32x4 kf[NDC], vf[NDC];
#pragma unroll
  for (int cc = 0; cc < NDC; ++cc) {
    const uint32_t off = ((uint32_t)mykey * D + 16 * cc + 8 * hh) * 2u;
    kf[cc] = buf_load16(rK, off);
    vf[cc] = buf_load16(rV, off);
  }
#pragma unroll
  for (int cc = 0; cc < NDC; ++cc) {
    settle(kf[cc]);
    settle(vf[cc]);
  }

  // Per-lane LDS offsets.  Row-major operands (S and dP): query row l32 of a
  // 32-row block, columns 16cc + 8hh.  Transposed operands (Q^T, dO^T for
  // dK^T, dV^T): as for the forward kernel's V^T reads, with queries as rows.
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

  f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dkacc[db][r] = 0.f;
      dvacc[db][r] = 0.f;
    }

  // One query tile.  MASKED: the tile overlaps this workgroup's keys on the
  // causal diagonal (per-wave skip of blocks wholly above it, element mask
  // on the rest); otherwise every (query, key) pair is visible and the body
  // is straight-line code, so the scheduler can overlap one block's softmax
  // arithmetic with the other block's MFMAs.
  auto tile = [&](const uint16_t* S0, int qs, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    constexpr int NQB = BR / 32;
    const uint16_t* Qs = S0;
    const uint16_t* dOs = S0 + TILE;
    const float* nls = reinterpret_cast<const float*>(S0 + 2 * TILE);
    const float* nds = nls + 64;
    // block qb holds queries that see some key of this wave
    auto live = [&](int qb) { return !MASKED || qs + qb * 32 + 31 >= wk0; };
    // lane: key `mykey`; register r of block qb: query
    // qs + 32qb + 8*(r/4) + 4*hh + r%4.  The accumulators start at that
    // query's -LSE/scale (S) and -Delta (dP): four consecutive registers are
    // four consecutive queries, one 16-byte LDS read each.
    f32x16 s[NQB], dp[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int qo = qb * 32 + 8 * g + 4 * hh;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(nls + qo);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(nds + qo);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[qb][4 * g + e] = l4[e];
          dp[qb][4 * g + e] = d4[e];
        }
      }
#pragma unroll
    for (int cc = 0; cc < NDC; ++cc)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
        if (live(qb)) {
          s[qb] = T::mfma(ld_lds16(Qs + qb * 32 * D + roff[cc]), kf[cc], s[qb]);
          dp[qb] = T::mfma(ld_lds16(dOs + qb * 32 * D + roff[cc]), vf[cc], dp[qb]);
        }
    // P = exp2(c (S - LSE/scale)), dS = P (dP - Delta)
    u32x4 pp[NQB][2], dsp[NQB][2];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const bool need_mask = MASKED && qs + qb * 32 < wk0 + 31;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int qo = qb * 32 + 8 * g + 4 * hh;
        float p[4], ds[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          float pv = fast_exp2(s[qb][r] * c);
          if (need_mask && qs + qo + e < mykey) pv = 0.f;
          p[e] = pv;
          ds[e] = pv * dp[qb][r];
        }
        pp[qb][g >> 1][2 * (g & 1)] = T::pack2(p[0], p[1]);
        pp[qb][g >> 1][2 * (g & 1) + 1] = T::pack2(p[2], p[3]);
        dsp[qb][g >> 1][2 * (g & 1)] = T::pack2(ds[0], ds[1]);
        dsp[qb][g >> 1][2 * (g & 1) + 1] = T::pack2(ds[2], ds[3]);
      }
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
      if (live(qb)) {
#pragma unroll
        for (int qc = 0; qc < 2; ++qc)
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const int rb = (qb * 32 + qc * 16) * D;
            const u32x4 ag =
                cat(ld_lds_tr(dOs + rb + toffs[db][0]), ld_lds_tr(dOs + rb + toffs[db][1]));
            dvacc[db] = T::mfma(ag, pp[qb][qc], dvacc[db]);
            const u32x4 aq =
                cat(ld_lds_tr(Qs + rb + toffs[db][0]), ld_lds_tr(Qs + rb + toffs[db][1]));
            dkacc[db] = T::mfma(aq, dsp[qb][qc], dkacc[db]);
          }
      }
  };
  // Causal: the first tiles (queries k0 .. k0+127) straddle the diagonal of
  // this workgroup's keys and take the masked body; every later tile is
  // wholly visible and runs the straight-line body.  All of them are
  // double-buffered, tile t in stage t % 2 (the diagonal spans an even
  // number of tiles, so the straight-line loop starts in stage 0).
  int t = 0;
  static_assert((kDkvKeys / BR) % 2 == 0, "the diagonal spans an even number of tiles");
  const int ndiag = CAUSAL ? min(ntiles, kDkvKeys / BR) : 0;
  wait_dma();
  __syncthreads();
  for (; t < ndiag; t += 2) {
    if (t + 1 < ntiles) dma(smem1, qstart + (t + 1) * BR);
    tile(smem0, qstart + t * BR, std::true_type());
    wait_dma();
    __syncthreads();
    if (t + 1 >= ndiag) {
      t += 1;
      break;
    }
    if (t + 2 < ntiles) dma(smem0, qstart + (t + 2) * BR);
    tile(smem1, qstart + (t + 1) * BR, std::true_type());
    wait_dma();
    __syncthreads();
  }
  if constexpr (D == 128 && !CAUSAL) {
    // One tile per iteration, the stage picked by parity.  With the MFMA
    // results kept in VGPRs (that instantiation is built in its own unit,
    // see fa_bwd_d128.hip) this form lets the register allocator keep the
    // dK/dV accumulators in place; unrolled by two it shuttled them between
    // register files on every tile.
    for (; t < ntiles; ++t) {
      const bool odd = (t - ndiag) & 1;
      if (t + 1 < ntiles) dma(odd ? smem0 : smem1, qstart + (t + 1) * BR);
      tile(odd ? smem1 : smem0, qstart + t * BR, std::false_type());
      wait_dma();
      __syncthreads();
    }
  } else {
    for (; t < ntiles; t += 2) {
      if (t + 1 < ntiles) dma(smem1, qstart + (t + 1) * BR);
      tile(smem0, qstart + t * BR, std::false_type());
      wait_dma();
      __syncthreads();
      if (t + 1 >= ntiles) break;
      if (t + 2 < ntiles) dma(smem0, qstart + (t + 2) * BR);
      tile(smem1, qstart + (t + 1) * BR, std::false_type());
      wait_dma();
      __syncthreads();
    }
  }

  if (mykey < N) {
    uint16_t* dKr = dK + base + (size_t)mykey * D;
    uint16_t* dVr = dV + base + (size_t)mykey * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + 8 * g + 4 * hh;
        u32x2 wk, wv;
        wk[0] = T::pack2(dkacc[db][4 * g] * scale, dkacc[db][4 * g + 1] * scale);
        wk[1] = T::pack2(dkacc[db][4 * g + 2] * scale, dkacc[db][4 * g + 3] * scale);
        wv[0] = T::pack2(dvacc[db][4 * g], dvacc[db][4 * g + 1]);
        wv[1] = T::pack2(dvacc[db][4 * g + 2], dvacc[db][4 * g + 3]);
        st_global8(dKr + d, wk);
        st_global8(dVr + d, wv);
      }
  }
}

template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(256, DkvTile<D>::MIN_WG)
bwd_dkdv_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                const float* __restrict__ nlse, const float* __restrict__ ndelta,
                uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int N, float c,
                float scale, int nkt, int total, int tile_major) {
  // Two stages in separate arrays, the loop unrolled by two: loads into one
  // stage provably never alias reads of the other (no spurious waits).
  __shared__ __attribute__((aligned(1024))) uint16_t smem0[dkv_stage_elems<D>()];
  __shared__ __attribute__((aligned(1024))) uint16_t smem1[dkv_stage_elems<D>()];
  dkdv_body<T, D, CAUSAL>(Q, K, V, dO, nlse, ndelta, dK, dV, N, c, scale, nkt, total,
                          tile_major, blockIdx.x, smem0, smem1);
}

// Launches the dK/dV kernel for one element type, head dimension and mask.
template <typename T, int D, bool CAUSAL>
static hipError_t dkdv(const BwdArgs& a) {
  const int nkt = (a.N + kDkvKeys - 1) / kDkvKeys;
  const int total = nkt * a.B * a.H;
  hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL>), dim3(total), dim3(256), 0, a.stream,
                     (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V,
                     (const uint16_t*)a.dO, a.nlse, a.ndelta, (uint16_t*)a.dK, (uint16_t*)a.dV,
                     a.N, a.scale * kLog2e, a.scale, nkt, total, tile_major(CAUSAL, nkt, total));
  return hipGetLastError();
}

}  // namespace fa
