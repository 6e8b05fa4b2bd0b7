// fa_fwd.hip -- forward kernels: O = softmax(scale Q K^T) V and LSE.
//
// Pages cited (by address and title):
//   [csdn]      adg.csdn.net/6a311d0d10ee7a33f27dee1b.html
//               "kk的大模型论文学习笔记 第8篇: FlashAttention"
//   [guanweilu] guanweilu.cn/article/445.html
//               "CUDA Kernel 级别的优化：Flash Attention 为什么比 PyTorch 原生实现快 5-10 倍"
//   [ijyty]     ijyty.com/news/1153309
//               "Flash Attention 技术原理让 Transformer 更快更高效"
//
// Method ([guanweilu] "FlashAttention 的三板斧", first and second technique;
// [csdn] "分块计算：厨房虽小，但够用" and "在线Softmax：分块了还能算对吗？"):
// a workgroup keeps one block of query rows resident and streams the key and
// value rows through on-chip memory one tile at a time.  Every row carries a
// running maximum m and a running sum l; when a tile raises m the partial
// output is scaled by exp(m_old - m_new), and the output is divided by l once
// after the last tile.  Scores and probabilities exist only in registers.
//
// 16-bit kernels, gfx950 design (fwd16_kernel: 4 waves, 128 query rows per
// workgroup; fwd16pp_kernel: 8 waves, 256 rows, described at its definition):
//   * each wave owns 32 query rows; its Q fragments stay in VGPRs for the
//     whole key loop (loaded once from HBM);
//   * K and V tiles are double-buffered in LDS, row-major with their 16-byte
//     chunks swizzled per row, and filled by direct global->LDS loads issued
//     a tile ahead; K fragments are 16-byte LDS reads, V^T fragments come
//     from the row-major V tile through transposing LDS reads; neither access
//     has bank conflicts;
//   * the score tile is computed transposed, S^T = K Q^T, so each lane holds
//     one query row: the row max needs one exchange between wave halves, the
//     row sum none until the epilogue, and the O^T accumulators of a lane all
//     belong to its row, so the rescale is a per-lane multiply;
//   * P^T leaves the S^T accumulators already in the B-operand layout of
//     O^T += V^T P^T, and the transposing reads hand each lane exactly the
//     keys its P registers hold;
//   * exp is exp2 with scale*log2(e) folded into the score: the score
//     accumulators start from a register block holding the reference, so a
//     weight is one multiply and one exp2; the reference maximum moves
//     lazily (see softmax_tile);
//   * causal: tiles wholly above a wave's rows are skipped per wave, the
//     workgroup stops at its last visible tile, only diagonal/tail tiles pay
//     for the mask, and the longest query blocks are launched first;
//   * an optional offset between query and key positions (partial attention
//     over blocks of a longer sequence) shifts all of these by a constant.
#include <hip/hip_runtime.h>

#include <float.h>
#include <math.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

template <int D>
struct FwdTile;
template <>
struct FwdTile<64> {
  static constexpr int BC = 128;  // keys per tile
};
template <>
struct FwdTile<128> {
  static constexpr int BC = 64;
};

constexpr int kFwdBR = 128;  // query rows per workgroup (4 waves x 32)
// Bound on a lane's partial row sum over one tile; it bounds every weight,
// and 2^15 keeps each weight finite when packed to fp16 (largest finite
// value 65504: a weight just under 2^16 would round to +inf).
constexpr float kSumLimit = 32768.f;

// Online softmax of one tile.  Exponentiates the scores against the
// reference maximum m (log2 units) and packs them as the B operand of
// O^T += V^T P^T (registers 8*half .. +7 of block kb are the 8 K-slots of
// reduction step 2*kb + half), adding the lane's weights to lpart.  The
// reference moves lazily: every weight is at most the lane's partial sum, so
// while no lane's sum exceeds kSumLimit the weights are safely bounded and m
// stays put.  Otherwise (always on a row's first tile, where m is still the
// lowest finite float) the wave takes the tile maximum, rescales O and l to
// it -- exact, since O and l always share the reference -- and exponentiates
// again.  The row maximum is therefore off the common path.
//
// SEED: the score accumulators started from the block `sd` holding -m/c in
// every register (an MFMA's C operand need not be its destination, so the
// block survives), i.e. s arrives as s - m/c and a weight costs a multiply
// and an exp2.  Until the row has a reference (m still the lowest float) sd
// is 0 and the wave takes the slow path, which also refreshes sd.
template <typename T, int NKB, int NDB, bool SEED>
__device__ __forceinline__ void softmax_tile(const f32x16 (&s)[NKB], u32x4 (&pk)[2 * NKB],
                                             float& m, float& lpart, f32x16 (&oacc)[NDB],
                                             float c, f32x16& sd) {
  // bias: added to c*s before the exp2 (unused on the seeded fast path)
  auto exp_pack = [&](float bias, auto fast) {
    constexpr bool FAST = decltype(fast)::value;
    float rs = -0.f;  // -0 + x == x for every x, so the first add folds away
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x0 = s[kb][8 * half + 2 * i], x1 = s[kb][8 * half + 2 * i + 1];
          const float p0 = fast_exp2(FAST ? x0 * c : fmaf(x0, c, bias));
          const float p1 = fast_exp2(FAST ? x1 * c : fmaf(x1, c, bias));
          rs += p0 + p1;
          pk[2 * kb + half][i] = T::pack2(p0, p1);
        }
    return rs;
  };
  const bool fresh = m == -FLT_MAX;  // no reference yet (then sd = 0)
  float rs = SEED ? exp_pack(0.f, std::true_type()) : exp_pack(-m, std::false_type());
  if (wave_any(!(rs <= kSumLimit) || (SEED && fresh))) {
    // the scores are c*s - meff in log2 units
    const float meff = SEED ? (fresh ? 0.f : m) : 0.f;
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    const float mnew = fmaxf(m, fmaf(max_halves(mx), c, meff));
    const float alpha = fast_exp2(m - mnew);  // 0 on the first tile
    lpart *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    rs = exp_pack(meff - mnew, std::false_type());
    m = mnew;
    if constexpr (SEED) {
      const float v = m == -FLT_MAX ? 0.f : -m / c;
#pragma unroll
      for (int r = 0; r < 16; ++r) sd[r] = v;
    }
  }
  lpart += rs;
}

// keep_if_le reads MFMA results from inside inline asm, where the compiler
// does not count the wait states a vector read of an MFMA destination needs.
// This block supplies them once per masked tile: 24 wait states (three
// s_nop 7), more than a 32x32 MFMA's result needs, and it takes the scores
// as operands so nothing that produces them can move past it.
template <int NKB>
__device__ __forceinline__ void mfma_result_guard(f32x16 (&s)[NKB]) {
  static_assert(NKB == 2 || NKB == 4, "score blocks per tile");
  if constexpr (NKB == 2)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s[0]), "+v"(s[1]));
  else
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+v"(s[0]), "+v"(s[1]), "+v"(s[2]), "+v"(s[3]));
}

// Sets the scores of invisible keys to -inf.  Register r of block kb holds
// key ts + 4hh + 32kb + 8(r/4) + r%4; keys at or past Nk, and (causal) past
// `last` (the lane's last visible key), are dropped.  The first form keeps
// each compare next to its select (see keep_if_le): left to the compiler,
// the compares of a 128-key tile (D = 64) or a causal tile are all hoisted
// and their masks spilled.  The 64-key unmasked-causal tiles (D = 128) keep
// the plain form, which compiles without spills.
template <bool CAUSAL, int NKB>
__device__ __forceinline__ void mask_tile(f32x16 (&s)[NKB], int ts, int Nk, int last, int hh) {
  if constexpr (CAUSAL || NKB == 4) {
    mfma_result_guard(s);
    const int lim = (CAUSAL ? min(Nk - 1, last) : Nk - 1) - ts - 4 * hh;
    const float ninf = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        s[kb][r] = keep_if_le(s[kb][r], lim, kb * 32 + 8 * (r >> 2) + (r & 3), ninf);
  } else {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (ts + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3) >= Nk) s[kb][r] = -INFINITY;
  }
}

template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(256, 2)
fwd16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
             const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
             float* __restrict__ LSE, int Nq, int Nk, int dlt, float c, int nqt,
             int total, int tile_major) {
  constexpr int BC = FwdTile<D>::BC;
  constexpr int TILE = BC * D;             // elements of one K or V tile
  constexpr int BLOCKS = TILE * 2 / 1024;  // 1 KiB blocks per tile
  constexpr int NKB = BC / 32;             // 32-key blocks per tile
  constexpr int NDC = D / 16;              // reduction steps of S^T = K Q^T
  constexpr int NDB = D / 32;              // 32-row blocks of O^T
  constexpr int NKC = BC / 16;             // reduction steps of O^T += V^T P^T
  static_assert(BLOCKS % 4 == 0, "blocks split evenly over 4 waves");

  // Two stages, each a K tile then a V tile, both row-major and swizzled.
  // Separate arrays (and a loop unrolled by two) let the compiler see that
  // the loads into one stage never alias the reads of the other, so it does
  // not wait for the prefetch before reading the current tile.
  __shared__ __attribute__((aligned(1024))) uint16_t smem0[2 * TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t smem1[2 * TILE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int l32 = lane & 31, hh = lane >> 5;

  int bh, qt;
  tile_of(blockIdx.x, total, nqt, tile_major, bh, qt);
  if (CAUSAL) qt = nqt - 1 - qt;  // longest rows first
  const int q0 = qt * kFwdBR;
  const int wq0 = q0 + wave * 32;
  const int myq = wq0 + l32;

  const size_t qbase = (size_t)bh * (size_t)Nq * D;
  const size_t kbase = (size_t)bh * (size_t)Nk * D;
  const auto rQ = make_rsrc(Q + qbase, (uint32_t)Nq * D * 2);
  const uint32_t kv_bytes = (uint32_t)Nk * D * 2;
  const i32x4 rK = rsrc_words(K + kbase, kv_bytes);  // direct-to-LDS sources
  const i32x4 rV = rsrc_words(V + kbase, kv_bytes);

  // B operand of S^T = K Q^T: lane (l32, hh) holds Q[myq][16c + 8hh .. +7]
  // (zeros past the last row).
  u32x4 qf[NDC];
#pragma unroll
  for (int cc = 0; cc < NDC; ++cc) qf[cc] = buf_load16(rQ, ((uint32_t)myq * D + 16 * cc + 8 * hh) * 2u);
#pragma unroll
  for (int cc = 0; cc < NDC; ++cc) settle(qf[cc]);

  // Per-lane LDS offsets (elements).  K operand: row l32 of a 32-key block,
  // columns 16cc + 8hh.  V^T operand via transposing reads: for d-block db
  // and half t, this lane addresses key row 8t + 4*(lane/32) + (lane%16)/4
  // of a 16-key chunk and d column 32db + 16*((lane/16)%2) + 4*(lane%4);
  // the read hands every lane d column 32db + lane%32 of keys
  // 16kc + 8t + 4*(lane/32) + {0,1,2,3}, exactly the keys whose P values sit
  // in its S^T accumulator registers 8*(kc%2) + 4t .. +3.
  int koff[NDC];
#pragma unroll
  for (int cc = 0; cc < NDC; ++cc) koff[cc] = toff<D>(l32, 16 * cc + 8 * hh);
  const int G = lane >> 4, a16 = lane & 15;
  int voff[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int t = 0; t < 2; ++t)
      voff[db][t] = toff<D>(8 * t + 4 * (G >> 1) + (a16 >> 2), 32 * db + 16 * (G & 1) + 4 * (a16 & 3));

  // Causal: key j is visible to query i iff j <= i + dlt.
  const int kend = CAUSAL ? max(0, min(Nk, q0 + kFwdBR + dlt)) : Nk;
  const int ntiles = (kend + BC - 1) / BC;

  // Direct global->LDS loads of one key tile into a stage (K then V).
  auto dma = [&](const uint16_t* Ks, int ts) {
#pragma unroll
    for (int i = 0; i < BLOCKS / 4; ++i) {
      const int b = wave_u + 4 * i;
      const uint32_t goff = dma_goff<D>(b, lane, ts);
      lds_dma16(rK, Ks + b * 512, goff);
      lds_dma16(rV, Ks + TILE + b * 512, goff);
    }
  };

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  // Reference maximum (log2 units) the exponents are taken against (moved
  // lazily, see softmax_tile), and the partial row sum over the keys this
  // lane holds.  It starts at the lowest finite float, not -inf: a row that
  // sees no key (possible with a position offset) then keeps weights
  // exp2(-inf) = 0 and rescale factors exp2(0) = 1 instead of NaN.
  float m = -FLT_MAX;
  float lpart = 0.f;
  constexpr bool SEED = true;  // seeded score accumulators (see softmax_tile)
  f32x16 sd;
#pragma unroll
  for (int r = 0; r < 16; ++r) sd[r] = 0.f;

  // MASKED: ragged tail or causal-diagonal tile (per-wave skip, element
  // mask); the others run straight-line code.
  auto tile = [&](const uint16_t* Ks, int ts, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    const uint16_t* Vs = Ks + TILE;
    if (!MASKED || !CAUSAL || ts <= wq0 + 31 + dlt) {
      // S^T[key][q] for the wave's 32 queries and the tile's BC keys.
      f32x16 s[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        if constexpr (SEED) {
          s[kb] = sd;
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
        }
      }
#pragma unroll
      for (int cc = 0; cc < NDC; ++cc)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          s[kb] = T::mfma(ld_lds16(Ks + kb * 32 * D + koff[cc]), qf[cc], s[kb]);
      if constexpr (D == 128) pipeline_reads<NDC * NKB, 1, 6, 0>();
      const bool need_mask = MASKED && ((ts + BC > Nk) || (CAUSAL && ts + BC - 1 > wq0 + dlt));
      if (need_mask) mask_tile<CAUSAL, NKB>(s, ts, Nk, myq + dlt, hh);
      u32x4 pk[NKC];  // P^T, the B operand of O^T += V^T P^T
      softmax_tile<T, NKB, NDB, SEED>(s, pk, m, lpart, oacc, c, sd);
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const uint16_t* vb = Vs + kc * 16 * D;
          const u32x4 a = cat(ld_lds_tr(vb + voff[db][0]), ld_lds_tr(vb + voff[db][1]));
          oacc[db] = T::mfma(a, pk[kc], oacc[db]);
        }
      if constexpr (D == 128) pipeline_reads<NKC * NDB, 2, 4, 1>();
    }
  };

  // Tiles visible to every row (no tail, not past the causal diagonal) come
  // first: straight-line body, double-buffered.  The rest (the causal
  // diagonal, a ragged tail) take the masked body.  The first of those is
  // prefetched like a full tile (during the last full one, or by the
  // prologue when there is none) and lands in stage nfull % 2; any further
  // one loads on its own (a loop that prefetched every masked tile measured
  // slower on short causal sequences).
  const int nfull = min(Nk / BC, CAUSAL ? max(0, q0 + dlt + 1) / BC : ntiles);
  int t = 0;
  if (ntiles > 0) dma(smem0, 0);
  wait_dma();
  __syncthreads();
  for (; t < nfull; t += 2) {
    // even tile in stage 0 while the odd one lands in stage 1, then swap
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
  if (t < ntiles) {
    // one copy of the masked body (a second one, per stage, made the
    // compiler spill registers at D = 128); no load is in flight here
    tile((t & 1) ? smem1 : smem0, t * BC, std::true_type());
    __syncthreads();
    ++t;
  }
  for (; t < ntiles; ++t) {
    dma(smem0, t * BC);
    wait_dma();
    __syncthreads();
    tile(smem0, t * BC, std::true_type());
    __syncthreads();
  }

  // Epilogue: one division by the full row sum, then bf16/f16 (RNE) stores.
  // A row with no visible key has ltot = 0: O = 0 and LSE = -inf.
  const float ltot = sum_halves(lpart);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  if (myq < Nq) {
    uint16_t* Oq = O + qbase + (size_t)myq * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = T::pack2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv);
        w[1] = T::pack2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
        st_global8(Oq + db * 32 + 8 * g + 4 * hh, w);
      }
    if (hh == 0) LSE[(size_t)bh * Nq + myq] = (m + log2f(ltot)) * kLn2;
  }
}

// Ping-pong variant for large grids: one workgroup = 8 waves = 256 query
// rows, one workgroup per CU.  Waves 0-3 (group A) and 4-7 (group B) pair up
// on the four SIMDs and run the same phase sequence one phase apart:
//   M(j): O^T += V^T P^T for tile j-1, then S^T = K Q^T for tile j  (MFMA)
//   X(j): mask, row max, rescale check, exp2, row sums, pack P      (VALU)
// Every phase ends at a workgroup barrier, so while one wave of a SIMD issues
// MFMAs the other runs its softmax: the matrix cores and the vector ALUs work
// at the same time instead of taking turns inside one wave.  K and V tiles
// have two LDS buffers each, filled by direct global->LDS loads issued two
// phases before they are read (K of tile j+1 and V of tile j at phase 2j).
// Group B, which is in its softmax phase whenever loads are issued, issues
// all of them, so the MFMA-phase waves start on their operands at once.
constexpr int kPpBR = 256;

template <typename T, int D, bool CAUSAL, int GROUP>
__device__ __forceinline__ void fwd16pp_body(const uint16_t* __restrict__ Q,
                                             const uint16_t* __restrict__ K,
                                             const uint16_t* __restrict__ V,
                                             uint16_t* __restrict__ O, float* __restrict__ LSE,
                                             int Nq, int Nk, int dlt, float c, int nqt,
                                             int total, int tile_major, uint16_t* kb0,
                                             uint16_t* kb1, uint16_t* vb0, uint16_t* vb1) {
  constexpr int BC = FwdTile<D>::BC;
  constexpr int TILE = BC * D;
  constexpr int BLOCKS = TILE * 2 / 1024;
  constexpr int NKB = BC / 32;
  constexpr int NDC = D / 16;
  constexpr int NDB = D / 32;
  constexpr int NKC = BC / 16;
  static_assert(BLOCKS % 4 == 0, "blocks split evenly over the 4 waves of group B");

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int l32 = lane & 31, hh = lane >> 5;

  int bh, qt;
  tile_of(blockIdx.x, total, nqt, tile_major, bh, qt);
  if (CAUSAL) qt = nqt - 1 - qt;  // longest rows first
  const int q0 = qt * kPpBR;
  const int wq0 = q0 + wave * 32;
  const int myq = wq0 + l32;

  const size_t qbase = (size_t)bh * (size_t)Nq * D;
  const size_t kbase = (size_t)bh * (size_t)Nk * D;
  const auto rQ = make_rsrc(Q + qbase, (uint32_t)Nq * D * 2);
  const uint32_t kv_bytes = (uint32_t)Nk * D * 2;
  const i32x4 rK = rsrc_words(K + kbase, kv_bytes);  // direct-to-LDS sources
  const i32x4 rV = rsrc_words(V + kbase, kv_bytes);

  // Loads of one tile, issued by the four waves of group B only.
  auto dma_tile = [&](const uint16_t* dst, const i32x4& r, int ts) {
#pragma unroll
    for (int i = 0; i < BLOCKS / 4; ++i) {
      const int b = (wave_u - 4) + 4 * i;
      lds_dma16(r, dst + b * 512, dma_goff<D>(b, lane, ts));
    }
  };
  // K of tile 0 travels while the queries load (one memory latency, not two).
  if (GROUP != 0) dma_tile(kb0, rK, 0);

  u32x4 qf[NDC];
#pragma unroll
  for (int cc = 0; cc < NDC; ++cc)
    qf[cc] = buf_load16(rQ, ((uint32_t)myq * D + 16 * cc + 8 * hh) * 2u);
#pragma unroll
  for (int cc = 0; cc < NDC; ++cc) settle(qf[cc]);

  // LDS offsets as in fwd16_kernel.
  int koff[NDC];
#pragma unroll
  for (int cc = 0; cc < NDC; ++cc) koff[cc] = toff<D>(l32, 16 * cc + 8 * hh);
  const int G = lane >> 4, a16 = lane & 15;
  int voff[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int t = 0; t < 2; ++t)
      voff[db][t] = toff<D>(8 * t + 4 * (G >> 1) + (a16 >> 2), 32 * db + 16 * (G & 1) + 4 * (a16 & 3));

  const int kend = CAUSAL ? max(0, min(Nk, q0 + kPpBR + dlt)) : Nk;
  const int ntiles = (kend + BC - 1) / BC;

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m = -FLT_MAX;  // reference max (log2 units), moved lazily; see fwd16_kernel
  constexpr bool SEED = true;
  f32x16 sd;  // seed of the score accumulators (see softmax_tile)
#pragma unroll
  for (int r = 0; r < 16; ++r) sd[r] = 0.f;
  float lpart = 0.f;    // partial row sum over this lane's keys
  f32x16 s[NKB];        // scores of the tile between its M and X phases
  u32x4 pk[NKC];        // probabilities between X(j) and M(j+1)

  auto active = [&](int j) { return !CAUSAL || j * BC <= wq0 + 31 + dlt; };

  // Independent accumulators are interleaved (reduction step outer) so
  // consecutive MFMAs never wait on each other's results.
  auto pv_block = [&](int j, const uint16_t* Vprev) {
    if (j >= 1 && j <= ntiles && active(j - 1)) {
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const uint16_t* vb = Vprev + kc * 16 * D;
          const u32x4 a = cat(ld_lds_tr(vb + voff[db][0]), ld_lds_tr(vb + voff[db][1]));
          oacc[db] = T::mfma(a, pk[kc], oacc[db]);
        }
      if constexpr (D == 128) pipeline_reads<NKC * NDB, 2, 3, 1>();
    }
  };
  auto s_block = [&](int j, const uint16_t* Kcur) {
    if (j < ntiles && active(j)) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        if constexpr (SEED) {
          s[kb] = sd;
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
        }
      }
#pragma unroll
      for (int cc = 0; cc < NDC; ++cc)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          s[kb] = T::mfma(ld_lds16(Kcur + kb * 32 * D + koff[cc]), qf[cc], s[kb]);
      if constexpr (D == 128) pipeline_reads<NDC * NKB, 1, 4, 0>();
    }
  };
  // At D = 128 the S^T block goes first (measured 0.1-1% faster there), at
  // D = 64 the PV block (S^T first measured 0.7% slower).
  // The wave in its matrix phase issues ahead of the other group's wave on
  // the same SIMD (wave priority 1 vs 0), so its MFMAs go first whenever
  // both are ready and the softmax work fills the gaps: measured -0.4 to
  // -0.6% at D = 128 (c5 unchanged); the converse priority and the same
  // scheme in the backward kernels measured neutral to 2% slower.
  auto phase_m = [&](int j, const uint16_t* Kcur, const uint16_t* Vprev) {
    __builtin_amdgcn_s_setprio(1);
    if constexpr (D == 128) {
      s_block(j, Kcur);
      pv_block(j, Vprev);
    } else {
      pv_block(j, Vprev);
      s_block(j, Kcur);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  auto phase_x = [&](int j) {
    if (j < 0 || j >= ntiles || !active(j)) return;
    const int ts = j * BC;
    const bool need_mask = (ts + BC > Nk) || (CAUSAL && ts + BC - 1 > wq0 + dlt);
    if (need_mask) mask_tile<CAUSAL, NKB>(s, ts, Nk, myq + dlt, hh);
    softmax_tile<T, NKB, NDB, SEED>(s, pk, m, lpart, oacc, c, sd);
  };

  // K of tile j+1 and V of tile j are loaded at slot 2j (two buffers each)
  // and first read at slot 2j+2; the odd slots' barriers wait for them.
  constexpr bool A = GROUP == 0;
  barrier_after_loads();
  // Slots 2t .. 2t+3 cover tiles t and t+1; group B runs one slot behind.
  for (int t = 0; t <= ntiles; t += 2) {
    if (!A && t + 1 < ntiles) dma_tile(kb1, rK, (t + 1) * BC);
    if (!A && t < ntiles) dma_tile(vb0, rV, t * BC);
    if (A) phase_m(t, kb0, vb1); else phase_x(t - 1);
    barrier_keep_loads();
    if (A) phase_x(t); else phase_m(t, kb0, vb1);
    barrier_after_loads();
    if (!A && t + 2 < ntiles) dma_tile(kb0, rK, (t + 2) * BC);
    if (!A && t + 1 < ntiles) dma_tile(vb1, rV, (t + 1) * BC);
    if (A) phase_m(t + 1, kb1, vb0); else phase_x(t);
    barrier_keep_loads();
    if (A) phase_x(t + 1); else phase_m(t + 1, kb1, vb0);
    barrier_after_loads();
  }

  // A row with no visible key has ltot = 0: O = 0 and LSE = -inf.
  const float ltot = sum_halves(lpart);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  if (myq < Nq) {
    uint16_t* Oq = O + qbase + (size_t)myq * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = T::pack2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv);
        w[1] = T::pack2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
        st_global8(Oq + db * 32 + 8 * g + 4 * hh, w);
      }
    if (hh == 0) LSE[(size_t)bh * Nq + myq] = (m + log2f(ltot)) * kLn2;
  }
}

template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(512, 1)
fwd16pp_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
               const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
               float* __restrict__ LSE, int Nq, int Nk, int dlt, float c, int nqt,
               int total, int tile_major) {
  constexpr int TILE = FwdTile<D>::BC * D;
  // Separate buffers with compile-time selection (the slot loop is unrolled
  // over two tiles): loads into one buffer never alias reads of another.
  __shared__ __attribute__((aligned(1024))) uint16_t kb0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t kb1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t vb0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t vb1[TILE];
  // Each group runs its own copy of the slot loop (no per-slot branch on it).
  if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 8) == 0)
    fwd16pp_body<T, D, CAUSAL, 0>(Q, K, V, O, LSE, Nq, Nk, dlt, c, nqt, total, tile_major, kb0,
                                  kb1, vb0, vb1);
  else
    fwd16pp_body<T, D, CAUSAL, 1>(Q, K, V, O, LSE, Nq, Nk, dlt, c, nqt, total, tile_major, kb0,
                                  kb1, vb0, vb1);
}

// fp32 kernel: true fp32 products on the vector ALUs (no reduced-precision
// matrix path), same online softmax.  Four lanes share one query row, each
// holding D/4 of its q and o; a workgroup covers 64 rows and streams 32-key
// tiles of K and V through LDS.
constexpr int kF32BR = 64;

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256)
fwd32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
             const float* __restrict__ V, float* __restrict__ O,
             float* __restrict__ LSE, int Nq, int Nk, int dlt, float c, int nqt,
             int total) {
  constexpr int BK = 32;
  constexpr int DP = D / 4;
  __shared__ __attribute__((aligned(16))) float Ks[BK * D];
  __shared__ __attribute__((aligned(16))) float Vs[BK * D];

  const int tid = threadIdx.x;
  const int qi = tid >> 2, part = tid & 3;
  const int logical = xcd_logical_block(blockIdx.x, total);
  const int bh = logical / nqt;
  int qt = logical - bh * nqt;
  if (CAUSAL) qt = nqt - 1 - qt;
  const int q0 = qt * kF32BR;
  const int myq = q0 + qi;
  const size_t qbase = (size_t)bh * (size_t)Nq * D;
  const size_t kbase = (size_t)bh * (size_t)Nk * D;

  float q[DP], o[DP];
#pragma unroll
  for (int e = 0; e < DP; ++e) {
    q[e] = myq < Nq ? Q[qbase + (size_t)myq * D + part * DP + e] : 0.f;
    o[e] = 0.f;
  }
  float m = -FLT_MAX, l = 0.f;  // finite start: rows that see no key stay NaN-free
  const int kend = CAUSAL ? max(0, min(Nk, q0 + kF32BR + dlt)) : Nk;

  for (int ts = 0; ts < kend; ts += BK) {
    __syncthreads();
    for (int i = tid; i < BK * D / 4; i += 256) {
      const int row = (i * 4) / D, col = (i * 4) % D;
      const int key = ts + row;
      f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (key < Nk) {
        kv = *reinterpret_cast<const f32x4*>(K + kbase + (size_t)key * D + col);
        vv = *reinterpret_cast<const f32x4*>(V + kbase + (size_t)key * D + col);
      }
      *reinterpret_cast<f32x4*>(Ks + row * D + col) = kv;
      *reinterpret_cast<f32x4*>(Vs + row * D + col) = vv;
    }
    __syncthreads();

    float s[BK];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < BK; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < DP; ++e) acc = fmaf(q[e], Ks[j * D + part * DP + e], acc);
      acc += __shfl_xor(acc, 1, 64);
      acc += __shfl_xor(acc, 2, 64);
      const int key = ts + j;
      if (key >= Nk || (CAUSAL && key > myq + dlt)) acc = -INFINITY;
      s[j] = acc;
      mx = fmaxf(mx, acc);
    }
    const float mnew = fmaxf(m, mx * c);
    const float alpha = fast_exp2(m - mnew);
    m = mnew;
    l *= alpha;
#pragma unroll
    for (int e = 0; e < DP; ++e) o[e] *= alpha;
#pragma unroll
    for (int j = 0; j < BK; ++j) {
      const float p = fast_exp2(fmaf(s[j], c, -mnew));
      l += p;
#pragma unroll
      for (int e = 0; e < DP; ++e) o[e] = fmaf(p, Vs[j * D + part * DP + e], o[e]);
    }
  }
  if (myq < Nq) {
    const float inv = l > 0.f ? 1.f / l : 0.f;  // no visible key: O = 0, LSE = -inf
#pragma unroll
    for (int e = 0; e < DP; ++e) O[qbase + (size_t)myq * D + part * DP + e] = o[e] * inv;
    if (part == 0) LSE[(size_t)bh * Nq + myq] = (m + log2f(l)) * kLn2;
  }
}

template <typename T, int D, bool CAUSAL>
static hipError_t launch16(const FwdArgs& a) {
  // Ping-pong kernel (one 256-row workgroup per CU at a time) when its grid
  // gives every CU at least two workgroups, or fills whole rounds of one per
  // CU; other grids run the 4-wave kernel, two 128-row workgroups per CU,
  // whose finer granularity evens out a partial last round.
  const int npp = (a.Nq + kPpBR - 1) / kPpBR;
  const long wpp = (long)npp * a.B * a.H;
  const int cus = cu_count();
  if (wpp >= 2L * cus || wpp % cus == 0) {
    const int total = npp * a.B * a.H;
    hipLaunchKernelGGL((fwd16pp_kernel<T, D, CAUSAL>), dim3(total), dim3(512), 0, a.stream,
                       (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V,
                       (uint16_t*)a.O, a.LSE, a.Nq, a.Nk, a.delta, a.scale * kLog2e, npp,
                       total, tile_major(CAUSAL, npp, total));
    return hipGetLastError();
  }
  const int nqt = (a.Nq + kFwdBR - 1) / kFwdBR;
  const int total = nqt * a.B * a.H;
  hipLaunchKernelGGL((fwd16_kernel<T, D, CAUSAL>), dim3(total), dim3(256), 0, a.stream,
                     (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V,
                     (uint16_t*)a.O, a.LSE, a.Nq, a.Nk, a.delta, a.scale * kLog2e, nqt, total,
                     tile_major(CAUSAL, nqt, total));
  return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t launch32(const FwdArgs& a) {
  const int nqt = (a.Nq + kF32BR - 1) / kF32BR;
  const int total = nqt * a.B * a.H;
  hipLaunchKernelGGL((fwd32_kernel<D, CAUSAL>), dim3(total), dim3(256), 0, a.stream,
                     (const float*)a.Q, (const float*)a.K, (const float*)a.V, (float*)a.O,
                     a.LSE, a.Nq, a.Nk, a.delta, a.scale * kLog2e, nqt, total);
  return hipGetLastError();
}

template <typename T>
static hipError_t dispatch16(const FwdArgs& a) {
  if (a.D == 64) return a.causal ? launch16<T, 64, true>(a) : launch16<T, 64, false>(a);
  return a.causal ? launch16<T, 128, true>(a) : launch16<T, 128, false>(a);
}

hipError_t launch_fwd(const FwdArgs& a) {
  switch (a.dtype) {
    case kF32:
      if (a.D == 64) return a.causal ? launch32<64, true>(a) : launch32<64, false>(a);
      return a.causal ? launch32<128, true>(a) : launch32<128, false>(a);
    case kBF16:
      return dispatch16<BF16>(a);
    default:
      return dispatch16<F16>(a);
  }
}

}  // namespace fa
