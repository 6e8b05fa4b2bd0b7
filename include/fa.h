/*
 * fa.h -- C ABI of libfa.so: FlashAttention fused exact attention on AMD
 * MI355X (gfx950), forward and backward.
 *
 * Pages cited (by address and title):
 *   [csdn]      adg.csdn.net/6a311d0d10ee7a33f27dee1b.html
 *               "kk的大模型论文学习笔记 第8篇: FlashAttention"
 *   [guanweilu] guanweilu.cn/article/445.html
 *               "CUDA Kernel 级别的优化：Flash Attention 为什么比 PyTorch 原生实现快 5-10 倍"
 *   [ijyty]     ijyty.com/news/1153309
 *               "Flash Attention 技术原理让 Transformer 更快更高效"
 *
 * Conventions shared by every entry point
 *   - Tensors are (batch B, heads H, sequence N, head dim D), contiguous,
 *     row stride D elements ([ijyty] "传统 Attention 的问题": the
 *     (batch, heads, seq_len, head_dim) layout).  Self-attention: queries and
 *     keys share N (fa_fwd_partial alone takes separate query and key
 *     lengths).  B * H * N <= 2^30 rows per tensor.
 *   - All tensor pointers are DEVICE pointers owned by the caller and must be
 *     16-byte aligned.  The compute entry points never allocate, free or
 *     synchronise; they only enqueue kernels on `stream` (a hipStream_t;
 *     NULL = the null stream) and return.  Device faults surface at the
 *     caller's next synchronisation.  The exception is the optional timing
 *     support at the end of this header: fa_timing_enable creates its event
 *     pool (2 x 8192 hipEvents, once per process) and, while timing is on,
 *     every launch records two events on its stream; fa_timing_read and
 *     fa_timing_enable synchronise on recorded events.
 *   - Grid limit: B * H * ceil(N / 64) < 2^23 (every launch stays below 2^32
 *     work-items), besides B * H * N <= 2^30.
 *   - Arguments are validated before any HIP call; on an error nothing is
 *     launched and no output is touched.
 *   - causal != 0 keeps key j for query i iff j <= i (diagonal included).
 *     The pages do not define the mask; this is the usual autoregressive one.
 *   - scale multiplies Q K^T before the softmax; it must lie in
 *     [2^-32, 2^32] (NaN rejected).  The pages use 1/sqrt(D) ([ijyty]
 *     naive_attention snippet); the range keeps scale * log2(e), which the
 *     kernels fold into one fp32 factor, a normal number.
 *   - Entry points are stateless and may be called from several host threads
 *     (the optional kernel timer below is guarded by a mutex).
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of Q, K, V, O, dO, dQ, dK, dV. */
typedef enum {
  FA_F32 = 0,   /* float32: checked at 1e-5 against the float64 oracle     */
  FA_BF16 = 1,  /* bfloat16 storage, fp32 accumulation, bf16 MFMA          */
  FA_F16 = 2    /* IEEE half storage, fp32 accumulation, f16 MFMA          */
} fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1,  /* null/misaligned pointer, B/H/N <= 0, N > 2^23, B*H*N > 2^30,
                               B*H*ceil(N/64) >= 2^23, bad scale, negative position            */
  FA_ERR_UNSUPPORTED = -2,  /* D not in {64, 128} or unknown dtype                         */
  FA_ERR_WORKSPACE = -3,    /* backward workspace missing or smaller than required          */
  FA_ERR_HIP = -4           /* a kernel launch failed (hipGetLastError after the launch)    */
} fa_status;

/*
 * fa_fwd -- O = softmax(scale * Q K^T) V, computed tile by tile with the
 * online softmax (per-row running max m and running sum l; the partial output
 * is rescaled whenever m grows and divided by l once at the end):
 * [guanweilu] "FlashAttention 的三板斧", first technique (tiling: S and P
 * live only on chip) and second technique (online softmax); [csdn]
 * "在线Softmax：分块了还能算对吗？".  The N x N score matrix never reaches HBM.
 *
 *   Q, K, V : [B, H, N, D] of `dtype`, read only.
 *   O       : [B, H, N, D] of `dtype`, written (bf16/f16: round to nearest even).
 *   LSE     : [B, H, N] float32, written: LSE_i = m_i + ln(l_i), the natural
 *             log of row i's softmax normaliser of the scaled, masked scores.
 *             The backward pass reads it to recompute P.
 *   D       : 64 or 128.  1 <= N <= 2^23 (ragged tails are masked).
 * Returns an fa_status.
 */
int fa_fwd(int dtype, int B, int H, int N, int D, float scale, int causal,
           const void* Q, const void* K, const void* V, void* O, float* LSE,
           void* stream);

/*
 * fa_fwd_partial -- attention of a block of Nq queries over a block of Nk
 * keys that may sit at other sequence positions: query row i is at position
 * q_pos + i, key row j at k_pos + j.  Same tiled online softmax as fa_fwd,
 * with the causal rule on positions: key j is kept for query i iff
 * k_pos + j <= q_pos + i.  The (O, LSE) pair it returns is the state the
 * online softmax carries ([guanweilu] "FlashAttention 的三板斧", second
 * technique), so results over disjoint key blocks combine exactly with
 * fa_merge -- the building block for splitting the keys of one sequence
 * over several passes or devices.  With Nq = Nk = N and q_pos = k_pos it
 * computes exactly what fa_fwd computes.
 *
 *   Q       : [B, H, Nq, D] of `dtype`, read only.
 *   K, V    : [B, H, Nk, D] of `dtype`, read only.
 *   O       : [B, H, Nq, D] of `dtype`, written.
 *   LSE     : [B, H, Nq] float32, written.  A query row that sees no key
 *             (causal, q_pos + i < k_pos) gets O = 0 and LSE = -inf.
 *   q_pos, k_pos : >= 0 and <= 2^62 (ignored when causal == 0).
 *   1 <= Nq, Nk <= 2^23; D and dtypes as fa_fwd.
 * Returns an fa_status.
 */
int fa_fwd_partial(int dtype, int B, int H, int Nq, int Nk, int D, float scale, int causal,
                   long long q_pos, long long k_pos, const void* Q, const void* K,
                   const void* V, void* O, float* LSE, void* stream);

/*
 * fa_merge -- combines, in place, two partial results for the same queries
 * over disjoint key sets (from fa_fwd_partial, fa_fwd or earlier merges):
 *   LSE <- ln(e^LSE + e^LSE_part),
 *   O   <- e^(LSE_old - LSE_new) O + e^(LSE_part - LSE_new) O_part,
 * the online-softmax update of [guanweilu] "FlashAttention 的三板斧",
 * second technique, applied to whole blocks.  A row whose two LSEs are both
 * -inf becomes O = 0, LSE = -inf.  Exact up to rounding: merging partials
 * over a split of the keys gives fa_fwd over all of them.
 *
 *   O       : [B, H, N, D] of `dtype`, read and written (partial a -> merged).
 *   LSE     : [B, H, N] float32, read and written.
 *   O_part  : [B, H, N, D] of `dtype`, read only (may equal O).
 *   LSE_part: [B, H, N] float32, read only.
 * Returns an fa_status.
 */
int fa_merge(int dtype, int B, int H, int N, int D, void* O, float* LSE, const void* O_part,
             const float* LSE_part, void* stream);

/*
 * Bytes of device workspace fa_bwd needs for this problem: two float32
 * [B, H, N] arrays, each padded to 256 bytes -- the per-row -Delta_i =
 * -dO_i . O_i and -LSE_i / scale.  Returns 0 for invalid or unsupported
 * problems (fp32 has no backward).
 */
size_t fa_bwd_workspace_bytes(int dtype, int B, int H, int N, int D, int causal);

/*
 * fa_bwd -- gradients of sum(O * dO) with respect to Q, K and V.  S and P are
 * recomputed on chip from Q, K and the saved LSE instead of being stored
 * ([csdn] "重计算：扔掉比存着更快"; [guanweilu] "FlashAttention 的三板斧",
 * third technique).  With P_ij = exp(scale q_i.k_j - LSE_i):
 *   dV = P^T dO,  dP = dO V^T,  Delta_i = dO_i . O_i,
 *   dS = P * (dP - Delta),  dQ = scale dS K,  dK = scale dS^T Q.
 * Three kernels on `stream`: Delta, then dK/dV (key tiles resident, query
 * tiles streamed), then dQ (query tiles resident, key tiles streamed).  No
 * atomics: the result is bit-for-bit repeatable.
 *
 *   Q, K, V, O, dO : [B, H, N, D] of `dtype`, read only (O and LSE from fa_fwd
 *                    with the same arguments).
 *   LSE            : [B, H, N] float32 from fa_fwd, read only.
 *   dQ, dK, dV     : [B, H, N, D] of `dtype`, written.
 *   workspace      : device buffer of at least fa_bwd_workspace_bytes(...)
 *                    bytes, 16-byte aligned, owned by the caller; contents on
 *                    entry are ignored.  FA_ERR_WORKSPACE if too small.
 */
int fa_bwd(int dtype, int B, int H, int N, int D, float scale, int causal,
           const void* Q, const void* K, const void* V, const void* O,
           const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
           void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_bwd_noalloc -- fa_bwd for callers that cannot allocate device memory
 * (code recorded into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results as fa_bwd, bit for bit, with the
 * workspace taken from a fixed scratch buffer the library holds on each GPU
 * (a device array of fa_bwd_noalloc_max_bytes() bytes, allocated when the
 * library's code is loaded on that GPU and kept until the process ends).
 * Allocates, frees and synchronises nothing.
 *
 *   Arguments as fa_bwd, without workspace and workspace_bytes.  The stream
 *   must belong to the current device (the one whose scratch is used):
 *   FA_ERR_INVALID_ARG otherwise.  Returns FA_ERR_WORKSPACE if
 *   fa_bwd_workspace_bytes(...) for the problem exceeds
 *   fa_bwd_noalloc_max_bytes() (B * H * N above 2^22 rows), and FA_ERR_HIP
 *   if the stream's device or the scratch's address cannot be looked up.
 *   All calls on one GPU share its scratch: calls that overlap in time on
 *   one GPU (several streams or threads) race and must be serialised by the
 *   caller.  The scratch keeps the last call's row statistics; every value a
 *   call reads is written earlier in the same call.
 */
int fa_bwd_noalloc(int dtype, int B, int H, int N, int D, float scale, int causal,
                   const void* Q, const void* K, const void* V, const void* O,
                   const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                   void* stream);

/* Size in bytes of the fixed scratch fa_bwd_noalloc uses on each GPU. */
size_t fa_bwd_noalloc_max_bytes(void);

/* Static English text for a status code. */
const char* fa_status_string(int status);

/* Library ABI version (increments on any signature change). */
int fa_version(void);

/*
 * Per-kernel device timing (measurement support, off by default).  While
 * enabled, every launch is bracketed by two hipEvents recorded on the launch
 * stream; fa_timing_read synchronises those events and returns, for one
 * kernel id, the number of timed launches and their summed duration in
 * milliseconds.  fa_timing_enable(1) also clears previous totals.  Events
 * come from a fixed pool of 8192 pairs created at the first enable (fa_fwd
 * and fa_fwd_partial both count as FA_KERNEL_FWD); launches beyond it are not
 * timed (counted in *dropped).  Reading drains the recorded pairs and frees
 * their slots once no launch holds one.  The records add a little host work
 * to each launch: time whole steps with timing off.
 */
enum {
  FA_KERNEL_FWD = 0,          /* forward kernel                          */
  FA_KERNEL_BWD_DELTA = 1,    /* backward: Delta = rowsum(dO * O)        */
  FA_KERNEL_BWD_DKDV = 2,     /* backward: dK, dV                        */
  FA_KERNEL_BWD_DQ = 3,       /* backward: dQ                            */
  FA_KERNEL_MERGE = 4,        /* fa_merge                                */
  FA_KERNEL_BWD_DKDV_DQ = 5,  /* backward: dK, dV and dQ in one launch,
                                 used instead of the two above for D = 64
                                 grids of at most 8 workgroups per CU     */
  FA_KERNEL_COUNT = 6
};
int fa_timing_enable(int on);
int fa_timing_read(int kernel_id, long long* launches, double* total_ms, long long* dropped);
const char* fa_kernel_name(int kernel_id);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
