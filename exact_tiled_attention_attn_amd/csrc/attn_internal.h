// Private interface between the C ABI entry points (attn_api.cpp) and the
// gfx950 kernels (attn_fwd.hip, attn_bwd.hip, attn_decode.hip).  Not
// installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstddef>

namespace attn {

// One forward problem, already validated by the entry point.
struct FwdProblem {
  const void *q, *k, *v;
  void *o;
  float *lse;
  int B, Hq, Hkv, N, d;
  float scale;
  int causal, window;  // window <= 0: none
};

// Kernel variants selectable through attn_fwd_ex.  Id 0 means "choose".
enum Variant : int {
  kAuto = 0,
  kWaves4 = 1,  // 4 waves (256 threads) per workgroup, 32 query rows per wave
  kWaves8 = 2,  // 8 waves (512 threads) per workgroup, 32 query rows per wave
  kPingPong = 3,  // 8 waves in two groups that alternate matrix and softmax phases
  kPersistent = 4,  // the same kernel, one workgroup per CU running several tiles
  kNumVariants = 5
};

const char *variant_name(int variant);

// Enqueue the forward kernel for `p` on `stream`.  Returns the HIP status of
// the launch call (hipSuccess when it was enqueued).
hipError_t launch_fwd(const FwdProblem &p, int variant, hipStream_t stream);

// One packed variable-length forward problem with the general mask,
// already validated.  Rows of sequence b: cu_seqlens[b] .. cu_seqlens[b+1]-1
// (device array) of each head's [total_rows][d] slice.
struct VarlenProblem {
  const void *q, *k, *v;
  void *o;
  float *lse;
  const int *cu_seqlens;
  int B, max_seqlen, total_rows, Hq, Hkv, d;
  float scale;
  int causal, window, radius, n_global;
};

hipError_t launch_fwd_varlen(const VarlenProblem &p, hipStream_t stream);

// One backward problem, already validated by the entry point.
struct BwdProblem {
  const void *q, *k, *v, *o, *dout;
  const float *lse;
  float *delta;  // workspace, B * Hq * N floats
  void *dq, *dk, *dv;
  int B, Hq, Hkv, N, d;
  float scale;
  int causal, window;  // window <= 0: none
};

// Enqueue the three backward kernels (Delta, dQ, dK/dV) for `p` on `stream`.
hipError_t launch_bwd(const BwdProblem &p, hipStream_t stream);

// FP8 packing: bf16 q, k, v -> e4m3 q8, k8 and the permuted transpose vt8,
// scales[0..2] (and the amax values in scales[3..5]).
struct Fp8Pack {
  const void *q, *k, *v;
  void *q8, *k8, *vt8;
  float *scales;
  int B, Hq, Hkv, N, d;
};
hipError_t launch_fp8_pack(const Fp8Pack &p, hipStream_t stream);

// FP8 forward over packed inputs.
struct Fp8Problem {
  const void *q8, *k8, *vt8;
  const float *scales;
  void *o;
  float *lse;
  int B, Hq, Hkv, N, d;
  float scale;
  int causal, window;
};
hipError_t launch_fwd_fp8(const Fp8Problem &p, hipStream_t stream);

// One paged decode problem, already validated by the entry point.
struct DecodeProblem {
  const void *q, *k_cache, *v_cache;
  const int *block_table, *seq_lens;
  void *o;
  float *lse;
  void *workspace;
  int B, Hq, Hkv, T, d, page_size, num_pages, max_pages, max_seq_len;
  float scale;
  int window;  // <= 0: none
};

// How the keys are split: nsplit ranges of `chunk` keys; the workspace
// holds part_o_floats partial outputs followed by part_lse_floats lse values.
struct DecodePlan {
  int nsplit, chunk;
  size_t part_o_floats, part_lse_floats;
};

// Deterministic in its arguments: the workspace size query and the launch
// agree.  All zero for a non-positive argument.
DecodePlan plan_decode(int B, int Hq, int Hkv, int T, int d, int page_size, int max_seq_len,
                       int window);

// Enqueue the split kernel and the merge kernel for `p` on `stream`.
hipError_t launch_decode(const DecodeProblem &p, const DecodePlan &plan, hipStream_t stream);

// Device address of the allocation-free decode's scratch array on the
// current device (looked up once per device).
hipError_t decode_noalloc_scratch(void **ptr);

}  // namespace attn
