/*
 * attn.h -- C ABI of the MI355X (gfx950) exact tiled attention: the forward
 * pass (dense, and packed variable-length with structured masks), its
 * gradients, and decode over a paged KV cache.
 *
 * Operation.  For every batch b, query head h and query row i
 *
 *     s_ij  = scale * <q[b,h,i,:], k[b,g(h),j,:]>
 *     o[b,h,i,:] = sum_j softmax_j(s_ij) v[b,g(h),j,:]      (visible j only)
 *     lse[b,h,i] = ln sum_j exp(s_ij)                        (visible j only)
 *
 * with g(h) = h / (Hq / Hkv).  Sources: the attention formula
 * softmax(QK^T / sqrt(d)) V of "Efficient Attention: FlashAttention, Sparse,
 * Linear" (section 45.2.1); the visibility rule of "Efficient attention: long
 * context and sub-quadratic variants" (sections "Sliding-window and local
 * attention" and "Implementation, twice": masked scores are -inf before the
 * softmax, row i sees i - window < j <= i); the KV-head map of "Attention
 * Mechanism Variants Beyond Self-Attention" (section "Multi-Query and
 * Grouped-Query Attention", repeat_interleave of the KV heads).  Key j is
 * visible from row i iff (causal == 0 || j <= i) && (window <= 0 ||
 * j > i - window).  The logsumexp output is the natural log over the *scaled*
 * scores, so that p_ij = exp(s_ij - lse_i).  The N x N score matrix is never
 * written to memory: it is computed tile by tile on chip with a running
 * (max, sum) softmax ("Efficient attention: long context and sub-quadratic
 * variants", section "FlashAttention: exact attention, IO-aware").
 *
 * Layout.  All tensors are dense, row-major, d innermost, in device memory:
 *     q   bf16 [B][Hq ][N][d]
 *     k   bf16 [B][Hkv][N][d]
 *     v   bf16 [B][Hkv][N][d]
 *     o   bf16 [B][Hq ][N][d]   written
 *     lse fp32 [B][Hq ][N]      written
 * bf16 is IEEE binary32 truncated to its upper 16 bits; o is rounded to
 * nearest even from the fp32 result.  Every pointer must be 16-byte aligned.
 * o and lse must not overlap q, k, v or each other.
 *
 * Ownership.  The caller allocates and owns every buffer.  The library
 * allocates no memory, keeps no global state and may be called from several
 * threads at once.
 *
 * Streams.  `stream` is a hipStream_t (NULL = the default stream).  The call
 * enqueues one kernel on it and returns without synchronising; o and lse are
 * valid once that stream's work has completed.
 *
 * Errors.  Arguments are checked before any HIP call; on a non-OK status
 * nothing is launched and o / lse are untouched.  B == 0 or N == 0 is a valid
 * empty problem: nothing is launched and null pointers are accepted.
 */
#ifndef EXACT_TILED_ATTN_H
#define EXACT_TILED_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_status {
  ATTN_OK = 0,
  /* null pointer (for a non-empty problem), negative size, Hq or Hkv < 1,
   * Hq % Hkv != 0, causal not 0 or 1, non-finite scale, unknown variant */
  ATTN_ERR_INVALID_ARG = 1,
  /* d not 64 or 128, window > 0 without causal, pointer not 16-byte aligned,
   * N > ATTN_MAX_N, or a variant that cannot run this problem */
  ATTN_ERR_UNSUPPORTED = 2,
  /* the HIP launch itself failed (hipLaunchKernel returned an error) */
  ATTN_ERR_LAUNCH = 3,
  /* attn_decode_paged_noalloc: the problem needs more scratch than the
   * library's fixed array (ATTN_DECODE_NOALLOC_MAX_BYTES), or the array's
   * device address could not be obtained */
  ATTN_ERR_NO_SCRATCH = 4
} attn_status_t;

/* Longest sequence accepted.  The kernels address one (batch, head) slice of
 * q, k or v with 32-bit byte offsets (at most N * d * 2 + one tile of slack),
 * which stays below 2^31 up to this length. */
#define ATTN_MAX_N (1 << 22)

/* Forward pass, default kernel variant for the shape.
 *   q, k, v   device pointers, layouts above
 *   o, lse    device pointers, written
 *   B         batch size (>= 0)
 *   Hq, Hkv   query / KV heads (>= 1, Hq % Hkv == 0; Hkv == Hq is plain
 *             multi-head attention, Hkv == 1 multi-query)
 *   N         sequence length of queries and keys (>= 0, <= ATTN_MAX_N)
 *   d         head dimension, 64 or 128
 *   scale     softmax scale (usually 1/sqrt(d)), applied in fp32
 *   causal    0 or 1
 *   window    <= 0: no window; >= 1: row i sees keys i-window < j <= i
 *             (requires causal == 1; window >= N is plain causal)
 *   stream    hipStream_t or NULL */
attn_status_t attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                       int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                       int window, void *stream);

/* Same operation with an explicit kernel variant (0 = the default choice,
 * 1 .. attn_num_variants()-1 = a specific tiling, see attn_variant_name).
 * For benchmarking and tests; every variant computes the same result up to
 * floating-point summation order. */
attn_status_t attn_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse,
                          int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                          int window, int variant, void *stream);

/* Forward over packed sequences of different lengths with structured masks.
 *
 * Block-diagonal packing: "Efficient attention: long context and
 * sub-quadratic variants" (section "Against the real libraries") names
 * xformers' BlockDiagonalMask among the masks that reach a kernel as
 * iteration bounds: sequence b is rows cu_seqlens[b] .. cu_seqlens[b+1]-1 of
 * every head's slice and attends only within itself.  Local plus global
 * attention (Longformer; same page, "Sliding-window and local attention",
 * and "Efficient Attention: FlashAttention, Sparse, Linear", 45.2.2): a
 * band of half-width `radius` around each token, and `n_global` global
 * tokens -- the first n_global positions of each sequence -- that attend
 * to, and are attended by, every token.  Within a sequence, row i sees key
 * j iff
 *     (causal == 0 || j <= i) &&
 *     (i < n_global || j < n_global ||
 *      ((window <= 0 || j > i - window) && (radius <= 0 || |i - j| <= radius)))
 * The kernel visits only the key tiles of the global keys and of the band.
 *
 *   q           bf16 [Hq][total_rows][d]     (head-major, sequences packed)
 *   k, v        bf16 [Hkv][total_rows][d]
 *   o           bf16 [Hq][total_rows][d]     written
 *   lse         fp32 [Hq][total_rows]        written
 *   cu_seqlens  int32 [B + 1], device memory, 0 = cu[0] <= ... <= cu[B] =
 *               total_rows, every length <= max_seqlen (not checked: the
 *               host never reads it)
 *   max_seqlen  host-side bound of the lengths (sizes the grid)
 *   radius, n_global  >= 0 (0: none); window as for attn_fwd
 * Errors as for attn_fwd (negative radius, n_global, total_rows -> invalid
 * argument; cu_seqlens not 4-byte aligned -> unsupported).  B == 0,
 * max_seqlen == 0 or total_rows == 0 launches nothing. */
attn_status_t attn_fwd_varlen(const void *q, const void *k, const void *v, void *o, float *lse,
                              const int *cu_seqlens, int B, int max_seqlen, int total_rows,
                              int Hq, int Hkv, int d, float scale, int causal, int window,
                              int radius, int n_global, void *stream);

/* FP8 forward.  "Efficient attention: long context and sub-quadratic
 * variants" (section "FlashAttention: exact attention, IO-aware") attaches
 * an FP8 path to FlashAttention-3.  Format: OCP FP8 E4M3 (bias 7, largest
 * finite 448, NaN = 0x7F / 0xFF, round to nearest even).  One power-of-two
 * scale per tensor: s = 2^e with e the smallest integer such that
 * max|x| <= 448 * 2^e, code = e4m3(x / s), value = code * s.
 *
 * attn_fp8_quantize: bf16 q, k, v (attn_fwd's layouts) ->
 *   q8   e4m3 [B][Hq][N][d]
 *   k8   e4m3 [B][Hkv][N][d]
 *   vt8  e4m3 [B][Hkv][d][Np], Np = N rounded up to a multiple of 64: V
 *        transposed, and within each 64-key block position p holds key
 *        32 (b / 16) + 8 ((b % 16) / 4) + 4 h + b % 4 with h = p / 32,
 *        b = p % 32 (the order the kernel's P^T operand holds the keys);
 *        positions of keys >= N hold 0.  attn_fp8_vt_bytes gives its size.
 *   scales  device float[6], written: scales[0..2] = s_q, s_k, s_v;
 *        scales[3..5] hold the amax values.
 * All pointers 16-byte aligned (scales 4-byte).  Four kernels on `stream`.
 *
 * attn_fwd_fp8: the attention of the dequantised tensors, with attn_fwd's
 * arguments otherwise (o bf16, lse fp32, causal, window, GQA).  Inside,
 * the weights are rounded to e4m3 for the P V product as 2^4 exp(s - m) with
 * a reference max m that moves only when a row's max exceeds it by more
 * than 4 log2 units (so they stay <= 2^8 < 448); S and O accumulate in
 * fp32, lse sums the unrounded weights. */
size_t attn_fp8_vt_bytes(int B, int Hkv, int N, int d);
attn_status_t attn_fp8_quantize(const void *q, const void *k, const void *v, void *q8, void *k8,
                                void *vt8, float *scales, int B, int Hq, int Hkv, int N, int d,
                                void *stream);
attn_status_t attn_fwd_fp8(const void *q8, const void *k8, const void *vt8, const float *scales,
                           void *o, float *lse, int B, int Hq, int Hkv, int N, int d, float scale,
                           int causal, int window, void *stream);

/* Backward pass: the gradients of a loss L with respect to q, k and v, given
 * dout = dL/do for the forward above.  "Efficient attention: long context
 * and sub-quadratic variants" (section "Against the real libraries") pairs
 * the exact forward with a recompute-based backward; the result is the
 * gradient of the forward definition, by the chain rule:
 *
 *     p_ij   = exp(s_ij - lse_i)                (recomputed from q, k, lse)
 *     D_i    = sum_c dout[i,c] * o[i,c]
 *     ds_ij  = p_ij * (<dout[i,:], v[j,:]> - D_i)
 *     dq[i]  = scale * sum_j ds_ij k[j]
 *     dk[j]  = scale * sum_i ds_ij q[i]         (summed over the query heads
 *     dv[j]  =         sum_i p_ij dout[i]        that share the KV head)
 *
 * (masked pairs have p = ds = 0).  The shared-KV-head sum follows from the
 * repeat_interleave of the KV heads ("Attention Mechanism Variants Beyond
 * Self-Attention", section "Multi-Query and Grouped-Query Attention").
 *
 *   q, k, v, o, lse   the forward's inputs and outputs (o bf16, lse fp32 as
 *                     written by attn_fwd for the same arguments)
 *   dout              bf16 [B][Hq][N][d]
 *   dq                bf16 [B][Hq][N][d]   written
 *   dk, dv            bf16 [B][Hkv][N][d]  written (every row, also rows
 *                                          no query sees)
 *   workspace         device memory of attn_bwd_workspace_size(B, Hq, N)
 *                     bytes, 16-byte aligned; holds D between the kernels,
 *                     contents on entry and exit unspecified
 *   the rest          as for attn_fwd
 * Outputs are rounded to nearest even from fp32 accumulators; the sums over
 * j and i are formed in fp32 with the products p * dout and ds * q, ds * k
 * rounded to bf16 (the matrix-core operand type) first.  dq, dk, dv and the
 * workspace must not overlap each other or any input.  The call enqueues
 * three kernels on `stream` and returns without synchronising.  Errors as for
 * attn_fwd (also for dout, dq, dk, dv and workspace); B == 0 or N == 0 is a
 * valid empty problem. */
attn_status_t attn_bwd(const void *q, const void *k, const void *v, const void *o,
                       const float *lse, const void *dout, void *dq, void *dk, void *dv,
                       void *workspace, int B, int Hq, int Hkv, int N, int d, float scale,
                       int causal, int window, void *stream);

/* Bytes of workspace attn_bwd needs: B * Hq * N * 4 (0 for an empty or
 * invalid shape).  The library never allocates it itself. */
size_t attn_bwd_workspace_size(int B, int Hq, int N);

/* Decode over a paged KV cache.  "Efficient attention: long context and
 * sub-quadratic variants" (section "FlashAttention: exact attention,
 * IO-aware") describes PagedAttention: the cache is stored in fixed-size
 * pages with a per-sequence page table, kernels gather K and V through the
 * table, sequences may share pages, and the result is exact attention.
 *
 * For sequence b with L = seq_lens[b] cached tokens, token j is slot
 * j % page_size of physical page block_table[b * max_pages_per_seq +
 * j / page_size].  Its T newest tokens are the queries: query t sits at
 * position pos = L - T + t and sees the cached keys j <= pos, and with
 * window > 0 only j > pos - window.  Query head h reads KV head
 * h / (Hq / Hkv).  Per (b, h, t):
 *     o   = sum_j softmax_j(scale * <q, k_j>) v_j,   lse = ln sum_j exp(...)
 * over the visible keys; a query that sees no key gets o = 0, lse = -inf.
 *
 *   q            bf16 [B][Hq][T][d]
 *   k_cache,     bf16 [num_pages][page_size][Hkv][d]
 *   v_cache
 *   block_table  int32 [B][max_pages_per_seq], physical page indices; an
 *                index outside [0, num_pages) reads as zero rows
 *   seq_lens     int32 [B], device memory, each in [0, max_seq_len] and
 *                covered by the table row (the host never reads it)
 *   o            bf16 [B][Hq][T][d]   written
 *   lse          fp32 [B][Hq][T]      written
 *   workspace    attn_decode_workspace_size(...) bytes of device memory,
 *                16-byte aligned, contents unspecified on entry and exit
 *   page_size    a power of two in [16, 4096]
 *   max_seq_len  host-side upper bound of seq_lens (decides the key split)
 *   scale        as for attn_fwd; window <= 0: none
 * Requires (Hq / Hkv) * T <= 1024 (the query heads of one KV head times the
 * new tokens, processed in blocks of 32 matrix-core columns that share each
 * K/V tile through the cache).  Keys are split into
 * ranges processed by separate workgroups; the partial results are merged
 * with lse = ln sum_s exp(lse_s), o = sum_s exp(lse_s - lse) o_s.  Two
 * kernels are enqueued on `stream`.  Errors as for attn_fwd (also: T < 1,
 * page size, heads x tokens > 1024, unaligned table or lens -> codes as
 * listed); B == 0 or max_seq_len == 0 launches nothing. */
attn_status_t attn_decode_paged(const void *q, const void *k_cache, const void *v_cache,
                                const int *block_table, const int *seq_lens, void *o, float *lse,
                                void *workspace, int B, int Hq, int Hkv, int T, int d,
                                int page_size, int num_pages, int max_pages_per_seq,
                                int max_seq_len, float scale, int window, void *stream);

/* Bytes of workspace attn_decode_paged needs for these arguments (0 for an
 * invalid or empty shape).  A window (> 0) shortens the span of keys the
 * split covers and so the workspace. */
size_t attn_decode_workspace_size(int B, int Hq, int Hkv, int T, int d, int page_size,
                                  int max_seq_len, int window);

/* Paged decode that allocates nothing, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  attn_decode_paged's operation and
 * arguments without the workspace: the split partials go to a scratch array
 * of ATTN_DECODE_NOALLOC_MAX_BYTES bytes that the library keeps in the
 * device memory of each GPU it runs on (its address is looked up on the
 * first call on a device, which must then be the current device; the array
 * lives until the process ends).  A problem whose
 * attn_decode_workspace_size(...) exceeds that returns ATTN_ERR_NO_SCRATCH
 * and launches nothing; otherwise errors as for attn_decode_paged.  The
 * call uses no allocating routine.  Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (other streams, other host
 * threads) race and must be serialized by the caller.  `stream` must belong
 * to the current device. */
#define ATTN_DECODE_NOALLOC_MAX_BYTES ((size_t)32 << 20)
attn_status_t attn_decode_paged_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                        const int *block_table, const int *seq_lens, void *o,
                                        float *lse, int B, int Hq, int Hkv, int T, int d,
                                        int page_size, int num_pages, int max_pages_per_seq,
                                        int max_seq_len, float scale, int window, void *stream);

/* Number of variant ids accepted by attn_fwd_ex (ids 0 .. n-1). */
int attn_num_variants(void);

/* Static, human-readable name of a variant id; "invalid" if out of range. */
const char *attn_variant_name(int variant);

/* Static, human-readable text for a status code. */
const char *attn_status_string(attn_status_t status);

/* What the HIP runtime reports for device `device`, for callers that build
 * a roofline denominator on the machine they run on (matrix-core peak =
 * compute units x peak engine clock x FLOP per CU and clock): compute units,
 * peak engine clock in kHz, memory clock in kHz and memory bus width in
 * bits.  A null pointer skips that field.  ATTN_ERR_INVALID_ARG for a device
 * id out of range, ATTN_ERR_LAUNCH when a runtime query fails; launches
 * nothing and leaves the current device unchanged. */
attn_status_t attn_device_info(int device, int *num_cus, int *max_clock_khz, int *mem_clock_khz,
                               int *mem_bus_bits);

/* ABI version of this header (incremented on any signature change). */
#define ATTN_ABI_VERSION 7
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_TILED_ATTN_H */
