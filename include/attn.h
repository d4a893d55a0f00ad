/*
 * attn.h -- C ABI of the MI355X (gfx950) exact tiled attention forward.
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
  ATTN_ERR_LAUNCH = 3
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

/* Number of variant ids accepted by attn_fwd_ex (ids 0 .. n-1). */
int attn_num_variants(void);

/* Static, human-readable name of a variant id; "invalid" if out of range. */
const char *attn_variant_name(int variant);

/* Static, human-readable text for a status code. */
const char *attn_status_string(attn_status_t status);

/* ABI version of this header (incremented on any signature change). */
#define ATTN_ABI_VERSION 1
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_TILED_ATTN_H */
