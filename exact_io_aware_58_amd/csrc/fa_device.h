// fa_device.h -- device-side building blocks shared by the forward and
// backward kernels: vector types, the gfx950 MFMA wrappers, 16-bit packing
// with round-to-nearest-even, wave64 lane exchange and the XCD-aware
// workgroup order.
//
// MFMA operand layout used throughout (v_mfma_f32_32x32x16_{bf16,f16},
// D[32x32] += A[32x16] B[16x32], one wave64):
//   A: lane l holds 8 consecutive K-slots of row m = l % 32, slot group l / 32
//   B: lane l holds 8 consecutive K-slots of column n = l % 32, same grouping
//   D: lane l, register r holds D[8*(r/4) + 4*(l/32) + r%4][l % 32]
// A and B pair K-slots identically, so a contraction is correct for any
// assignment of the reduction index to (l/32, slot) as long as both operands
// use the same one; the kernels rely on that to feed an accumulator straight
// back in as the next product's operand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- element traits: 16-bit storage types with an fp32-accumulating MFMA ----
struct BF16 {
  using vec8 = bf16x8;
  __device__ static inline f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // two floats -> packed pair, round to nearest even (v_cvt_pk_bf16_f32)
  __device__ static inline uint32_t pack2(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
  __device__ static inline float to_float(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
};

struct F16 {
  using vec8 = f16x8;
  __device__ static inline f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static inline uint32_t pack2(float lo, float hi) {
    f16x2 v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
  __device__ static inline float to_float(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
  }
};

// ---- lane exchange ----
// Combine a value with the one held by lane l ^ 32 (the other wave half)
// using v_permlane32_swap: after the swap one result register holds the
// lower half twice and the other the upper half twice, so max/sum of the two
// gives every lane the pairwise result whichever half the swap moves.
__device__ inline float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 2^x on the transcendental unit (v_exp_f32).  Results below 2^-126 flush to
// zero, which only drops softmax weights smaller than 1e-38 of the row max.
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Makes the wave wait here until `v` has arrived.  For operands loaded once
// before a loop: left alone, the compiler may issue such loads after the
// prologue's barrier, and then waits on the memory counter inside the loop,
// where the count also covers the direct-to-LDS prefetches in flight -- every
// tile would stall until its prefetch landed.  The empty asm consumes the
// value, so the wait happens once, here.
template <typename V>
__device__ __forceinline__ void settle(const V& v) {
  asm volatile("" ::"v"(v));
}

// True on every lane when any lane of the wave has `pred` set.
__device__ inline bool wave_any(bool pred) { return __builtin_amdgcn_ballot_w64(pred) != 0; }

// s when off <= lim, else `ninf` (-inf held in a VGPR); `off` is a
// compile-time constant after unrolling.  The compare and the select sit in
// one asm block, so masking a tile never keeps dozens of lane masks alive in
// scalar registers at once (left to itself the compiler hoists all the
// compares of a tile and spills their masks).  s_nop 1: the wait states a
// VALU write of VCC needs before a VALU reads it as a lane mask.
__device__ __forceinline__ float keep_if_le(float s, int lim, int off, float ninf) {
  float r;
  asm("v_cmp_gt_i32_e32 vcc, %2, %1\n\ts_nop 1\n\tv_cndmask_b32_e32 %0, %3, %4, vcc"
      : "=v"(r)
      : "v"(lim), "i"(off), "v"(s), "v"(ninf)
      : "vcc");
  return r;
}

// ---- buffer loads ----
// A raw buffer resource over one (batch, head) slab: loads whose byte offset
// is at or past `bytes` return zeros instead of touching memory, which masks
// ragged tails without branches.  Word 3 = 0x00020000 is the gfx9 data format
// for untyped 32-bit dwords.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ inline u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}
__device__ inline float buf_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}

// ---- memory helpers ----
__device__ inline u32x4 ld_global16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ inline void st_global8(void* p, u32x2 v) {
  *reinterpret_cast<u32x2*>(p) = v;
}
__device__ inline u32x4 ld_lds16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Select the 16-bit element j (0..7) of a 16-byte vector.
__device__ inline uint32_t elem16(u32x4 v, int j) {
  uint32_t w = v[j >> 1];
  return (j & 1) ? (w >> 16) : (w & 0xffffu);
}

// ---- swizzled row-major LDS tiles ----
// A tile of rows of D 16-bit elements is stored densely (row stride D), with
// the 16-byte chunk c of row r placed at chunk position c ^ g(r).  gfx950 LDS
// has 64 banks of 4 bytes (256 bytes per cycle).  g is chosen so that
//  * 16 lanes reading the same chunk of 16 consecutive rows (a 16-byte MFMA
//    operand read, one row per lane) hit 16 distinct 16-byte bank groups, and
//  * the 32 lanes of a transposing read (ds_read_b64_tr_b16: 4 consecutive
//    rows x 64 aligned bytes each) cover all 256 bytes of the banks once;
// both are conflict-free.  g only uses row bits 0..3, so a row offset that is
// a multiple of 16 leaves the swizzle unchanged (offsets stay additive).
// The layout is dense in 1 KiB blocks, which is what the direct
// global->LDS loads write (64 lanes x 16 bytes, lane l at byte 16*l).
template <int D>
struct Swz;
template <>
struct Swz<128> {  // 16 chunks per 256-byte row
  __device__ static inline int g(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
};
template <>
struct Swz<64> {  // 8 chunks per 128-byte row, two rows per bank cycle
  __device__ static inline int g(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }
};
// element offset of (row r, column col) inside a swizzled tile
template <int D>
__device__ inline int toff(int r, int col) {
  return r * D + (((col >> 3) ^ Swz<D>::g(r)) << 3) + (col & 7);
}

typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ inline lds_void* to_lds(const void* p) {
  return (lds_void*)((__attribute__((address_space(3))) char*)(p));
}

// Buffer resource as four dwords (for inline assembly): 48-bit base, stride
// 0, `bytes` records, gfx9 dword format.  Loads past `bytes` return zeros.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ inline i32x4 rsrc_words(const void* base, uint32_t bytes) {
  const unsigned long long p = (unsigned long long)base;
  return i32x4{(int)(uint32_t)p, (int)((uint32_t)(p >> 32) & 0xffffu), (int)bytes, 0x00020000};
}

// One 1 KiB block of a swizzled tile straight from global memory into LDS:
// lane l fetches 16 bytes at byte offset `goff` of the buffer and the
// hardware writes them to lds_block + 16*l (lds_block is wave-uniform, passed
// in M0).  Offsets past the buffer's end write zeros.  Written as inline
// assembly so that the compiler does not track these LDS writes itself: it
// would otherwise make LDS reads of *other* buffers wait for every load in
// flight.  The kernels order them explicitly (vmcnt waits before the
// barriers that publish a buffer); the "memory" clobber keeps other memory
// accesses from moving across.  M0 is only used this way in these kernels.
// An LDS-direct load reading M0 needs one wait state after the scalar write
// of M0 (the s_nop 0); the compiler cannot insert it inside the asm.
__device__ inline void lds_dma16(const i32x4& r, const uint16_t* lds_block, uint32_t goff) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)(
      (__attribute__((address_space(3))) const uint16_t*)lds_block);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(m0)), "v"(goff), "s"(r)
               : "memory");
}
// Same for 4-byte elements (64 lanes x 4 bytes = 256 bytes).
__device__ inline void lds_dma4(const i32x4& r, const void* lds_block, uint32_t goff) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)(
      (__attribute__((address_space(3))) const char*)lds_block);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(m0)), "v"(goff), "s"(r)
               : "memory");
}

// Global byte offset lane `lane` must fetch for 1 KiB block `b` of a tile
// whose first row is global row `row0`.
template <int D>
__device__ inline uint32_t dma_goff(int b, int lane, int row0) {
  constexpr int CPR = D / 8, RPB = 512 / D;
  const int row = b * RPB + lane / CPR;
  const int chunk = (lane % CPR) ^ Swz<D>::g(row);
  return ((uint32_t)(row0 + row) * D + chunk * 8) * 2u;
}

// Wait until this wave's direct-to-LDS loads have landed (vmcnt = 0).
__device__ inline void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup barrier that does not wait for outstanding direct-to-LDS loads.
// __syncthreads() is a release/acquire fence plus s_barrier, and the fence
// makes every wave drain its vector-memory counter, i.e. wait for prefetches
// meant to stay in flight across the barrier.  Here the wave's own LDS reads
// are drained (lgkmcnt = 0: nothing it still reads can be overwritten by a
// load another wave issues after the barrier) and the barrier is emitted as
// an instruction the compiler may not move memory operations across.
__device__ inline void barrier_keep_loads() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt/expcnt untouched
  asm volatile("s_barrier" ::: "memory");
}
// Barrier after this wave's loads have landed (vmcnt = lgkmcnt = 0).
__device__ inline void barrier_after_loads() {
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

// 64-bit transposing LDS read: within each 16-lane group, lane j receives
// element j%4 of the 8-byte chunks addressed by lanes j/4, 4+j/4, 8+j/4 and
// 12+j/4 (one element from each of four rows).
__device__ inline u32x2 ld_lds_tr(const uint16_t* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)to_lds(p));
  return __builtin_bit_cast(u32x2, v);
}
__device__ inline u32x4 cat(u32x2 lo, u32x2 hi) { return u32x4{lo[0], lo[1], hi[0], hi[1]}; }

// ---- instruction scheduling ----
// Scheduling hint for a block of NM MFMAs that each consume R LDS reads:
// issue the reads of the first AHEAD MFMAs, then alternate one MFMA with the
// reads of the MFMA AHEAD places later.  Left to itself the compiler issues
// each read just before its MFMA; where only two or four accumulator chains
// are in flight every MFMA then waits for LDS latency.
template <int NM, int R, int AHEAD, int GROUP_ID>
__device__ __forceinline__ void pipeline_reads() {
  constexpr int kDsRead = 0x100, kMfma = 0x008;
  __builtin_amdgcn_sched_group_barrier(kDsRead, R * AHEAD, GROUP_ID);
#pragma unroll
  for (int i = 0; i < NM - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, GROUP_ID);
    __builtin_amdgcn_sched_group_barrier(kDsRead, R, GROUP_ID);
  }
  __builtin_amdgcn_sched_group_barrier(kMfma, AHEAD, GROUP_ID);
}

// ---- workgroup order ----
// Workgroups are dealt round-robin to the 8 XCDs (blockIdx.x % 8).  Remap so
// that each XCD receives one contiguous range of logical tiles: tiles of the
// same (batch, head) then share that XCD's L2 while they stream the same K/V.
__device__ inline int xcd_logical_block(int pid, int total) {
  constexpr int kXcd = 8;
  int q = total / kXcd, r = total % kXcd;
  int x = pid % kXcd, local = pid / kXcd;
  return x * q + (x < r ? x : r) + local;
}

// (batch*head, tile) of workgroup `pid` in a grid of `total` = heads x
// `ntile` workgroups.  Head-major (the default) goes through
// xcd_logical_block, so a head's tiles share one XCD's L2.  Tile-major puts
// the tile index outermost: consecutive workgroups are the same tile of
// different heads, and since workgroups are dealt to the XCDs in dispatch
// order, every tile rank is spread over all XCDs.  Causal grids with few
// tiles per head but several rounds of workgroups use it so that the
// longest tiles of all heads run first (head-major would interleave long
// and short ones).
__device__ inline void tile_of(int pid, int total, int ntile, int tile_major, int& bh, int& t) {
  if (tile_major) {
    const int nbh = total / ntile;
    t = pid / nbh;
    bh = pid - t * nbh;
  } else {
    const int logical = xcd_logical_block(pid, total);
    bh = logical / ntile;
    t = logical - bh * ntile;
  }
}

}  // namespace fa
