// C ABI entry points: argument validation, then the kernel launches.
//
// Validation runs before any HIP call, so a rejected call launches nothing
// and leaves o / lse untouched.  The rules follow the problem statement in
// include/attn.h: the visibility rule j <= i (causal) and i - w < j (window)
// of "Efficient attention: long context and sub-quadratic variants"
// (sections "Sliding-window and local attention", "Implementation, twice"),
// where the window is only defined together with the causal mask, and the
// KV-head map h / (Hq / Hkv) of "Attention Mechanism Variants Beyond
// Self-Attention" (section "Multi-Query and Grouped-Query Attention"), whose
// integer head ratio needs Hq to be a multiple of Hkv.

#include <cmath>
#include <cstdint>

#include "attn.h"
#include "attn_internal.h"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

attn_status_t validate(const attn::FwdProblem &p, int variant) {
  if (variant < 0 || variant >= attn::kNumVariants) return ATTN_ERR_INVALID_ARG;
  if (p.B < 0 || p.N < 0) return ATTN_ERR_INVALID_ARG;
  if (p.Hq < 1 || p.Hkv < 1 || p.Hq % p.Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (p.causal != 0 && p.causal != 1) return ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(p.scale)) return ATTN_ERR_INVALID_ARG;
  if (p.d != 64 && p.d != 128) return ATTN_ERR_UNSUPPORTED;
  if (p.window > 0 && p.causal == 0) return ATTN_ERR_UNSUPPORTED;
  if (p.N > ATTN_MAX_N) return ATTN_ERR_UNSUPPORTED;
  if (p.B == 0 || p.N == 0) return ATTN_OK;  // empty problem: pointers unused
  if (!p.q || !p.k || !p.v || !p.o || !p.lse) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(p.q) || !aligned16(p.k) || !aligned16(p.v) || !aligned16(p.o) ||
      !aligned16(p.lse))
    return ATTN_ERR_UNSUPPORTED;
  // Grid size: B * Hq * ceil(N / 32) workgroup-rows must fit a 32-bit grid.
  const int64_t rows = static_cast<int64_t>(p.B) * p.Hq * ((static_cast<int64_t>(p.N) + 31) / 32);
  if (rows > (int64_t{1} << 31) - 1) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

attn_status_t validate_bwd(const attn::BwdProblem &p) {
  const attn::FwdProblem f{p.q, p.k, p.v, const_cast<void *>(p.o), const_cast<float *>(p.lse),
                           p.B, p.Hq, p.Hkv, p.N, p.d, p.scale, p.causal, p.window};
  const attn_status_t st = validate(f, attn::kAuto);
  if (st != ATTN_OK) return st;
  if (p.B == 0 || p.N == 0) return ATTN_OK;
  if (!p.dout || !p.dq || !p.dk || !p.dv || !p.delta) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(p.dout) || !aligned16(p.dq) || !aligned16(p.dk) || !aligned16(p.dv) ||
      !aligned16(p.delta))
    return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

attn_status_t validate_varlen(const attn::VarlenProblem &p) {
  if (p.B < 0 || p.max_seqlen < 0 || p.total_rows < 0 || p.radius < 0 || p.n_global < 0)
    return ATTN_ERR_INVALID_ARG;
  if (p.Hq < 1 || p.Hkv < 1 || p.Hq % p.Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (p.causal != 0 && p.causal != 1) return ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(p.scale)) return ATTN_ERR_INVALID_ARG;
  if (p.d != 64 && p.d != 128) return ATTN_ERR_UNSUPPORTED;
  if (p.window > 0 && p.causal == 0) return ATTN_ERR_UNSUPPORTED;
  if (p.max_seqlen > ATTN_MAX_N) return ATTN_ERR_UNSUPPORTED;
  if (p.B == 0 || p.max_seqlen == 0 || p.total_rows == 0) return ATTN_OK;
  if (!p.q || !p.k || !p.v || !p.o || !p.lse || !p.cu_seqlens) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(p.q) || !aligned16(p.k) || !aligned16(p.v) || !aligned16(p.o) ||
      !aligned16(p.lse) || (reinterpret_cast<uintptr_t>(p.cu_seqlens) & 3u) != 0)
    return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

bool pow2_in(int x, int lo, int hi) { return x >= lo && x <= hi && (x & (x - 1)) == 0; }

attn_status_t validate_decode(const attn::DecodeProblem &p, bool need_workspace = true) {
  if (p.B < 0 || p.T < 1 || p.num_pages < 0 || p.max_pages < 0 || p.max_seq_len < 0)
    return ATTN_ERR_INVALID_ARG;
  if (p.Hq < 1 || p.Hkv < 1 || p.Hq % p.Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(p.scale)) return ATTN_ERR_INVALID_ARG;
  if (p.d != 64 && p.d != 128) return ATTN_ERR_UNSUPPORTED;
  if (!pow2_in(p.page_size, 16, 4096)) return ATTN_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(p.Hq / p.Hkv) * p.T > 1024) return ATTN_ERR_UNSUPPORTED;
  if (p.max_seq_len > ATTN_MAX_N) return ATTN_ERR_UNSUPPORTED;
  if (p.B == 0 || p.max_seq_len == 0) return ATTN_OK;  // nothing to read or write
  if (!p.q || !p.k_cache || !p.v_cache || !p.block_table || !p.seq_lens || !p.o || !p.lse ||
      (need_workspace && !p.workspace))
    return ATTN_ERR_INVALID_ARG;
  if (p.num_pages < 1 || p.max_pages < 1) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(p.q) || !aligned16(p.k_cache) || !aligned16(p.v_cache) || !aligned16(p.o) ||
      !aligned16(p.lse) || (need_workspace && !aligned16(p.workspace)) ||
      (reinterpret_cast<uintptr_t>(p.block_table) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(p.seq_lens) & 3u) != 0)
    return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

}  // namespace

extern "C" {

attn_status_t attn_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse,
                          int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                          int window, int variant, void *stream) {
  attn::FwdProblem p{q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, window};
  const attn_status_t st = validate(p, variant);
  if (st != ATTN_OK) return st;
  if (B == 0 || N == 0) return ATTN_OK;
  if (p.window >= N) p.window = 0;  // a window covering every key is plain causal
  if (p.window < 0) p.window = 0;
  const hipError_t e = attn::launch_fwd(p, variant, static_cast<hipStream_t>(stream));
  if (e == hipErrorInvalidValue) return ATTN_ERR_UNSUPPORTED;
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

attn_status_t attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                       int Hq, int Hkv, int N, int d, float scale, int causal, int window,
                       void *stream) {
  return attn_fwd_ex(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, window, attn::kAuto,
                     stream);
}

attn_status_t attn_fwd_varlen(const void *q, const void *k, const void *v, void *o, float *lse,
                              const int *cu_seqlens, int B, int max_seqlen, int total_rows,
                              int Hq, int Hkv, int d, float scale, int causal, int window,
                              int radius, int n_global, void *stream) {
  attn::VarlenProblem p{q,  k,  v,   o,   lse,   cu_seqlens, B,      max_seqlen, total_rows,
                        Hq, Hkv, d, scale, causal, window, radius, n_global};
  const attn_status_t st = validate_varlen(p);
  if (st != ATTN_OK) return st;
  if (B == 0 || max_seqlen == 0 || total_rows == 0) return ATTN_OK;
  if (p.window >= max_seqlen) p.window = 0;
  if (p.radius >= max_seqlen) p.radius = 0;
  if (p.n_global > max_seqlen) p.n_global = max_seqlen;
  const hipError_t e = attn::launch_fwd_varlen(p, static_cast<hipStream_t>(stream));
  if (e == hipErrorInvalidValue) return ATTN_ERR_UNSUPPORTED;
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

size_t attn_fp8_vt_bytes(int B, int Hkv, int N, int d) {
  if (B <= 0 || Hkv <= 0 || N <= 0 || (d != 64 && d != 128)) return 0;
  const size_t np = (static_cast<size_t>(N) + 63) / 64 * 64;
  return static_cast<size_t>(B) * static_cast<size_t>(Hkv) * static_cast<size_t>(d) * np;
}

attn_status_t attn_fp8_quantize(const void *q, const void *k, const void *v, void *q8, void *k8,
                                void *vt8, float *scales, int B, int Hq, int Hkv, int N, int d,
                                void *stream) {
  const attn::FwdProblem f{q, k, v, q8, scales, B, Hq, Hkv, N, d, 1.0f, 0, 0};
  attn_status_t st = validate(f, attn::kAuto);
  if (st != ATTN_OK) return st;
  if (B == 0 || N == 0) return ATTN_OK;
  if (!k8 || !vt8) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(k8) || !aligned16(vt8)) return ATTN_ERR_UNSUPPORTED;
  const attn::Fp8Pack p{q, k, v, q8, k8, vt8, scales, B, Hq, Hkv, N, d};
  const hipError_t e = attn::launch_fp8_pack(p, static_cast<hipStream_t>(stream));
  if (e == hipErrorInvalidValue) return ATTN_ERR_UNSUPPORTED;
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

attn_status_t attn_fwd_fp8(const void *q8, const void *k8, const void *vt8, const float *scales,
                           void *o, float *lse, int B, int Hq, int Hkv, int N, int d, float scale,
                           int causal, int window, void *stream) {
  attn::FwdProblem f{q8, k8, vt8, o, lse, B, Hq, Hkv, N, d, scale, causal, window};
  attn_status_t st = validate(f, attn::kAuto);
  if (st != ATTN_OK) return st;
  if (B == 0 || N == 0) return ATTN_OK;
  if (!scales) return ATTN_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(scales) & 3u) != 0) return ATTN_ERR_UNSUPPORTED;
  attn::Fp8Problem p{q8, k8, vt8, scales, o, lse, B, Hq, Hkv, N, d, scale, causal, window};
  if (p.window >= N) p.window = 0;
  if (p.window < 0) p.window = 0;
  const hipError_t e = attn::launch_fwd_fp8(p, static_cast<hipStream_t>(stream));
  if (e == hipErrorInvalidValue) return ATTN_ERR_UNSUPPORTED;
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

size_t attn_bwd_workspace_size(int B, int Hq, int N) {
  if (B <= 0 || Hq <= 0 || N <= 0) return 0;
  return static_cast<size_t>(B) * static_cast<size_t>(Hq) * static_cast<size_t>(N) * sizeof(float);
}

attn_status_t attn_bwd(const void *q, const void *k, const void *v, const void *o,
                       const float *lse, const void *dout, void *dq, void *dk, void *dv,
                       void *workspace, int B, int Hq, int Hkv, int N, int d, float scale,
                       int causal, int window, void *stream) {
  attn::BwdProblem p{q,  k,  v,  o, dout, lse, static_cast<float *>(workspace), dq, dk, dv, B, Hq,
                     Hkv, N, d, scale, causal, window};
  const attn_status_t st = validate_bwd(p);
  if (st != ATTN_OK) return st;
  if (B == 0 || N == 0) return ATTN_OK;
  if (p.window >= N) p.window = 0;
  if (p.window < 0) p.window = 0;
  const hipError_t e = attn::launch_bwd(p, static_cast<hipStream_t>(stream));
  if (e == hipErrorInvalidValue) return ATTN_ERR_UNSUPPORTED;
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

size_t attn_decode_workspace_size(int B, int Hq, int Hkv, int T, int d, int page_size,
                                  int max_seq_len, int window) {
  if (Hkv < 1 || Hq < 1 || Hq % Hkv != 0 || (d != 64 && d != 128)) return 0;
  const attn::DecodePlan plan =
      attn::plan_decode(B, Hq, Hkv, T, d, page_size, max_seq_len, window);
  return (plan.part_o_floats + plan.part_lse_floats) * sizeof(float);
}

attn_status_t attn_decode_paged(const void *q, const void *k_cache, const void *v_cache,
                                const int *block_table, const int *seq_lens, void *o, float *lse,
                                void *workspace, int B, int Hq, int Hkv, int T, int d,
                                int page_size, int num_pages, int max_pages_per_seq,
                                int max_seq_len, float scale, int window, void *stream) {
  attn::DecodeProblem p{q,  k_cache, v_cache, block_table, seq_lens,          o,
                        lse, workspace, B,      Hq,          Hkv,               T,
                        d,  page_size, num_pages, max_pages_per_seq, max_seq_len, scale,
                        window};
  const attn_status_t st = validate_decode(p);
  if (st != ATTN_OK) return st;
  if (B == 0 || max_seq_len == 0) return ATTN_OK;
  if (p.window < 0) p.window = 0;
  const attn::DecodePlan plan =
      attn::plan_decode(B, Hq, Hkv, T, d, page_size, max_seq_len, p.window);
  const hipError_t e = attn::launch_decode(p, plan, static_cast<hipStream_t>(stream));
  if (e == hipErrorInvalidValue) return ATTN_ERR_UNSUPPORTED;
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

attn_status_t attn_decode_paged_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                        const int *block_table, const int *seq_lens, void *o,
                                        float *lse, int B, int Hq, int Hkv, int T, int d,
                                        int page_size, int num_pages, int max_pages_per_seq,
                                        int max_seq_len, float scale, int window, void *stream) {
  attn::DecodeProblem p{q,  k_cache, v_cache, block_table, seq_lens,          o,
                        lse, nullptr, B,      Hq,          Hkv,               T,
                        d,  page_size, num_pages, max_pages_per_seq, max_seq_len, scale,
                        window};
  const attn_status_t st = validate_decode(p, false);
  if (st != ATTN_OK) return st;
  if (B == 0 || max_seq_len == 0) return ATTN_OK;
  if (p.window < 0) p.window = 0;
  const attn::DecodePlan plan =
      attn::plan_decode(B, Hq, Hkv, T, d, page_size, max_seq_len, p.window);
  if ((plan.part_o_floats + plan.part_lse_floats) * sizeof(float) > ATTN_DECODE_NOALLOC_MAX_BYTES)
    return ATTN_ERR_NO_SCRATCH;
  if (attn::decode_noalloc_scratch(&p.workspace) != hipSuccess) return ATTN_ERR_NO_SCRATCH;
  const hipError_t e = attn::launch_decode(p, plan, static_cast<hipStream_t>(stream));
  if (e == hipErrorInvalidValue) return ATTN_ERR_UNSUPPORTED;
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int attn_num_variants(void) { return attn::kNumVariants; }

const char *attn_variant_name(int variant) { return attn::variant_name(variant); }

const char *attn_status_string(attn_status_t status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported problem";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
    case ATTN_ERR_NO_SCRATCH: return "problem exceeds the allocation-free scratch";
  }
  return "unknown status";
}

attn_status_t attn_device_info(int device, int *num_cus, int *max_clock_khz, int *mem_clock_khz,
                               int *mem_bus_bits) {
  if (device < 0) return ATTN_ERR_INVALID_ARG;
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess) return ATTN_ERR_LAUNCH;
  if (device >= n) return ATTN_ERR_INVALID_ARG;
  const struct {
    int *out;
    hipDeviceAttribute_t attr;
  } q[] = {{num_cus, hipDeviceAttributeMultiprocessorCount},
           {max_clock_khz, hipDeviceAttributeClockRate},
           {mem_clock_khz, hipDeviceAttributeMemoryClockRate},
           {mem_bus_bits, hipDeviceAttributeMemoryBusWidth}};
  for (const auto &e : q) {
    if (!e.out) continue;
    if (hipDeviceGetAttribute(e.out, e.attr, device) != hipSuccess) return ATTN_ERR_LAUNCH;
  }
  return ATTN_OK;
}

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

}  // extern "C"
