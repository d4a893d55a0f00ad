// gfx950 (MI355X, CDNA4) exact attention backward: dQ, dK, dV.
//
// What is computed: the gradient of the forward definition (masked scores
// -inf before the softmax, lse the natural logsumexp of the scaled scores)
// with respect to Q, K and V for an upstream gradient dO, by the chain rule;
// "Efficient attention: long context and sub-quadratic variants", section
// "Against the real libraries", names this recompute-based backward next to
// the exact forward.  Per (batch, query head), K and V those of its KV head:
//   P     = exp(sigma * Q K^T - lse)        (recomputed from the forward's lse)
//   Delta = rowsum(dO * O)
//   dP    = dO V^T,  dS = P * (dP - Delta)
//   dV    = P^T dO,  dQ = sigma dS K,  dK = sigma dS^T Q
// and a KV head shared by G query heads receives the sum of their dK, dV.
//
// Three kernels, one workgroup barrier per tile, no atomics:
// * attn_bwd_delta_kernel: Delta for every query row into the caller's
//   workspace (4 lanes per row).
// * attn_bwd_dq_kernel: workgroups over query tiles, as the forward.  A wave
//   owns 32 query rows and holds Q^T and dO^T as MFMA B operands; per 64-key
//   tile it computes S^T = K Q^T and dP^T = V dO^T (one query per lane, so lse
//   and Delta are lane scalars), dS^T, and dQ^T += K^T dS^T with K^T read by
//   transposing LDS reads.
// * attn_bwd_dkdv_kernel: workgroups over (batch, KV head, 128 keys).  A wave
//   owns 32 keys and holds K^T and V^T as B operands; per 32-query block of
//   every query head of the group it computes S = Q K^T and dP = dO V^T (one
//   key per lane: only this layout lets P and dS be the B operands of the
//   contractions over queries), then dV^T += dO^T P and dK^T += Q^T dS with
//   dO^T and Q^T read by transposing LDS reads.  lse and Delta vary per
//   accumulator row here and are read from LDS next to the Q and dO tiles;
//   Delta is folded in by starting the dP accumulator at -Delta.
// Tiles read both ways (K in the dQ kernel, Q and dO in the dK/dV kernel)
// are staged into LDS twice, once at the b128 stride and once at the
// transposed-read stride, so every read is bank-conflict-free.

#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "attn_device.h"
#include "attn_internal.h"

namespace attn {
namespace {

using namespace dev;

constexpr int kBN = 64;      // keys per tile (dQ kernel), query rows per tile (dK/dV kernel)

struct BwdParams {
  const uint16_t *q, *k, *v, *o, *dout;
  const float *lse;
  float *delta;   // [B][Hq][N]
  uint16_t *dq, *dk, *dv;
  int B, Hq, Hkv, N;
  int G;          // Hq / Hkv
  int groups;     // dQ kernel: Hq / P
  int nq;         // dQ kernel: query tiles per head group
  int total;      // workgroups of the kernel being launched
  int nkt;        // key tiles of 64 (dQ kernel) = query tiles of 64 (dK/dV kernel)
  int nkb;        // dK/dV kernel: key blocks per (batch, KV head)
  float c;        // scale * log2(e): P = exp2(c <q, k> - lse * log2(e))
  float scale;    // dQ = scale * dS K, dK = scale * dS^T Q
  int causal;
  int window;     // 0: none
};

// ---------------------------------------------------------------------------
// Delta = rowsum(dO * O): four lanes per row, D / 4 values each.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_delta_kernel(BwdParams prm) {
  const long long rows = (long long)prm.B * prm.Hq * prm.N;
  const long long row = (long long)blockIdx.x * 64 + (threadIdx.x >> 2);
  const int part = threadIdx.x & 3;
  float acc = 0.0f;
  if (row < rows) {
    const uint16_t *op = prm.o + row * D + part * (D / 4);
    const uint16_t *gp = prm.dout + row * D + part * (D / 4);
#pragma unroll
    for (int c8 = 0; c8 < D / 32; ++c8) {
      const bf16x8 a = *(const bf16x8 *)(op + 8 * c8);
      const bf16x8 b = *(const bf16x8 *)(gp + 8 * c8);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)a[e], (float)b[e], acc);
    }
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  if (part == 0 && row < rows) prm.delta[row] = acc;
}

// One thread's share of staging a 64-row tile of two [rows][D] tensors into
// LDS: kLoads 16-byte chunks per tensor (chunk n covers tile row
// (n * NT + tid) / kCh), rows past the end read as zero.
template <int D, int NT>
struct PairStage {
  using st = Stride<D>;
  static constexpr int kLoads = kBN * st::kCh / NT;
  static_assert(kLoads * NT == kBN * st::kCh, "tile must split evenly over the threads");
  u32x4 a[kLoads], b[kLoads];

  // Issues the loads only: nothing here consumes the data, so the wave
  // does not wait for it before the tile computed meanwhile.
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                       int row0, int tid) {
#pragma unroll
    for (int n = 0; n < kLoads; ++n) {
      const int off = row0 * st::kRowB + (n * NT + tid) * 16;
      a[n] = __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0);
      b[n] = __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0);
    }
  }
  // Tensor a into tile a1 (stride S1) and tile a2 (stride S2); tensor b into
  // tile b1 (stride S1) and, when kB2, tile b2 (stride S2).
  template <int S1, int S2, bool kB2>
  __device__ __forceinline__ void store(lchar *a1, lchar *a2, lchar *b1, lchar *b2, int tid) const {
    constexpr int kRowsPerLoad = NT / st::kCh;
    const int r0 = tid / st::kCh, p = tid % st::kCh;
#pragma unroll
    for (int n = 0; n < kLoads; ++n) {
      const int r = r0 + n * kRowsPerLoad;
      *(lds_u32x4_t *)(a1 + r * S1 + p * 16) = a[n];
      *(lds_u32x4_t *)(a2 + r * S2 + p * 16) = a[n];
      *(lds_u32x4_t *)(b1 + r * S1 + p * 16) = b[n];
      if constexpr (kB2) *(lds_u32x4_t *)(b2 + r * S2 + p * 16) = b[n];
    }
  }
};

// ---------------------------------------------------------------------------
// dQ: workgroups over query tiles (NW waves x 32 rows, P heads packed for GQA
// as in the forward), loop over 64-key tiles with one barrier each.
// ---------------------------------------------------------------------------
template <int D, int NW, int P>
__global__ __launch_bounds__(NW * 64, 2) void attn_bwd_dq_kernel(BwdParams prm) {
  using st = Stride<D>;
  constexpr int kRows = 32 * NW / P;
  constexpr int kKb = kBN * st::kB128;   // K tile for b128 reads
  constexpr int kKt = kBN * st::kTr;     // K tile for transposed reads
  constexpr int kVb = kBN * st::kB128;   // V tile for b128 reads
  constexpr int kSet = kKb + kKt + kVb;

  __shared__ __attribute__((aligned(1024))) char smem[2 * kSet];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;

  const Task tk = make_task<P, kRows, kBN>(prm, wave);
  const int N = prm.N;
  const __amdgpu_buffer_rsrc_t rs_k = make_rsrc(prm.k + tk.kv_slice * D, (uint32_t)N * D * 2);
  const __amdgpu_buffer_rsrc_t rs_v = make_rsrc(prm.v + tk.kv_slice * D, (uint32_t)N * D * 2);

  // Q^T and dO^T B operands: lane holds query row qw0 + l32, d = 16kk + 8hh ..
  const int row = tk.qw0 + l32;
  bf16x8 qf[st::kKSteps], of[st::kKSteps];
#pragma unroll
  for (int kk = 0; kk < st::kKSteps; ++kk) {
    qf[kk] = row_frag<D>(prm.q + tk.q_slice * D, row, N, 16 * kk + 8 * hh, false);
    of[kk] = row_frag<D>(prm.dout + tk.q_slice * D, row, N, 16 * kk + 8 * hh, false);
  }
  const float lse2 = row < N ? prm.lse[tk.q_slice + row] * kLog2e : 0.0f;
  const float delta = row < N ? prm.delta[tk.q_slice + row] : 0.0f;
#pragma unroll
  for (int kk = 0; kk < st::kKSteps; ++kk) {
    settle(qf[kk]);
    settle(of[kk]);
  }
  settle(lse2);
  settle(delta);
  const float c = prm.c;

  const int kb_lane = b128_lane_off<st::kB128>(lane);
  const int kt_lane = tr_lane_off<st::kTr>(lane);

  f32x16 dqacc[st::kDB];
#pragma unroll
  for (int i = 0; i < st::kDB; ++i) dqacc[i] = f32x16{};

  PairStage<D, NW * 64> stage;
  auto put = [&](lchar *set) {
    stage.template store<st::kB128, st::kTr, false>(set, set + kKb, set + kKb + kKt, set, tid);
  };
  if (tk.wg_lo < tk.wg_hi) {
    stage.load(rs_k, rs_v, tk.wg_lo * kBN, tid);
    put((lchar *)smem);
  }
  __syncthreads();

  // edge mask: key j is visible from this lane's row iff
  // (unsigned)(j - m_lo) < m_span
  const int m_lo = prm.window > 0 ? max(0, row - prm.window + 1) : 0;
  const int m_span = row < N ? (prm.causal ? row : N - 1) - m_lo + 1 : 0;

  auto compute = [&](int t, const lchar *set, auto &&store_next) {
    const lchar *kb = set + kb_lane;
    const lchar *kt = set + kKb + kt_lane;
    const lchar *vb = set + kKb + kKt + kb_lane;
    const int j0 = t * kBN;
    const bool need_mask = edge_tile(prm.causal, prm.window, j0, kBN, tk.qw0, N);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      // the next tile's LDS stores go out between the two key blocks, when
      // its loads have had half the tile to land
      if (rb == 1) store_next();
      // S^T and dP^T (32 keys x 32 queries)
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int kk = 0; kk < st::kKSteps; ++kk) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b128_frag<st::kB128>(kb, kk, rb), qf[kk], s,
                                                    0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b128_frag<st::kB128>(vb, kk, rb), of[kk],
                                                     dp, 0, 0, 0);
      }
      // register r holds key j0 + 32 rb + 8 (r / 4) + 4 hh + r % 4
      f32x16 p;
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -lse2));
      if (need_mask) {
        const int base = j0 + 32 * rb + 4 * hh - m_lo;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          p[r] = (unsigned)(base + 8 * (r >> 2) + (r & 3)) < (unsigned)m_span ? p[r] : 0.0f;
      }
      bf16x8 dsf[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) dsf[r >> 3][r & 7] = (__bf16)(p[r] * (dp[r] - delta));
      // dQ^T += K^T dS^T
#pragma unroll
      for (int db = 0; db < st::kDB; ++db) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          dqacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<st::kTr>(kt, db, rb, tt),
                                                              dsf[tt], dqacc[db], 0, 0, 0);
        }
      }
    }
  };

  lchar *const set0 = (lchar *)smem;
  lchar *const set1 = (lchar *)smem + kSet;
  auto step = [&](int t, const lchar *cur, lchar *next) {
    const bool more = t + 1 < tk.wg_hi;
    if (more) stage.load(rs_k, rs_v, (t + 1) * kBN, tid);
    auto store_next = [&]() {
      if (more) put(next);
    };
    if (t >= tk.w_lo && t < tk.w_hi) {
      compute(t, cur, store_next);
    } else {
      store_next();
    }
    __syncthreads();
  };
  for (int t = tk.wg_lo; t < tk.wg_hi; t += 2) {
    step(t, set0, set1);
    if (t + 1 < tk.wg_hi) step(t + 1, set1, set0);
  }

  if (row < N) store_rows<D>(prm.dq + tk.q_slice * D, row, hh, dqacc, prm.scale);
}

// ---------------------------------------------------------------------------
// dK, dV: workgroups over (batch, KV head, 32 * NW keys); loop over the query
// heads of the group and their 64-row query tiles, one barrier each.
// ---------------------------------------------------------------------------
template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 1) void attn_bwd_dkdv_kernel(BwdParams prm) {
  using st = Stride<D>;
  constexpr int kKeys = 32 * NW;         // keys per workgroup
  constexpr int kTb = kBN * st::kB128;   // tile for b128 reads
  constexpr int kTt = kBN * st::kTr;     // tile for transposed reads
  // set: Q (b128), Q (tr), dO (b128), dO (tr), lse * log2(e), Delta
  constexpr int kQb = 0, kQt = kTb, kOb = kTb + kTt, kOt = 2 * kTb + kTt;
  constexpr int kLse = 2 * kTb + 2 * kTt, kDel = kLse + 4 * kBN;
  constexpr int kSet = kDel + 4 * kBN;

  __shared__ __attribute__((aligned(1024))) char smem[2 * kSet];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int N = prm.N;

  const int logical = xcd_remap(blockIdx.x, prm.total);
  const int kblk = logical % prm.nkb;   // the lowest key blocks see the most queries
  const int bk = logical / prm.nkb;
  const int b = bk / prm.Hkv, kvh = bk % prm.Hkv;
  const int k0 = kblk * kKeys;
  const int kw0 = k0 + 32 * wave;       // this wave's first key
  const int key = kw0 + l32;            // this lane's key
  const size_t kv_slice = (size_t)(b * prm.Hkv + kvh) * N;

  // K^T and V^T B operands: lane holds key row `key`, d = 16kk + 8hh ..
  bf16x8 kf[st::kKSteps], vf[st::kKSteps];
#pragma unroll
  for (int kk = 0; kk < st::kKSteps; ++kk) {
    kf[kk] = row_frag<D>(prm.k + kv_slice * D, key, N, 16 * kk + 8 * hh, false);
    vf[kk] = row_frag<D>(prm.v + kv_slice * D, key, N, 16 * kk + 8 * hh, false);
  }
#pragma unroll
  for (int kk = 0; kk < st::kKSteps; ++kk) {
    settle(kf[kk]);
    settle(vf[kk]);
  }

  // query tiles the workgroup's keys and this wave's keys are seen from
  auto qrange = [&](int j_lo, int j_hi, int &lo, int &hi) {  // keys [j_lo, j_hi)
    lo = prm.causal ? j_lo / kBN : 0;
    hi = prm.nkt;
    if (prm.window > 0) hi = min(prm.nkt, (min(N, j_hi - 1 + prm.window) - 1) / kBN + 1);
  };
  int qlo, qhi, wlo, whi;
  qrange(k0, min(N, k0 + kKeys), qlo, qhi);
  if (kw0 < N) {
    qrange(kw0, min(N, kw0 + 32), wlo, whi);
  } else {
    wlo = whi = 0;
  }
  const int per_head = max(qhi - qlo, 0);
  const int steps = prm.G * per_head;

  const int qb_lane = b128_lane_off<st::kB128>(lane);
  const int qt_lane = tr_lane_off<st::kTr>(lane);
  const float c = prm.c;

  f32x16 dkacc[st::kDB], dvacc[st::kDB];
#pragma unroll
  for (int i = 0; i < st::kDB; ++i) {
    dkacc[i] = f32x16{};
    dvacc[i] = f32x16{};
  }

  PairStage<D, NW * 64> stage;
  // threads 0 .. kBN-1 carry lse * log2(e) of the tile's rows, threads
  // kBN .. 2 kBN-1 their Delta (the two LDS arrays are adjacent)
  const bool row_val = tid < 2 * kBN;
  const float *const val_src = tid < kBN ? prm.lse : prm.delta;
  const float val_mul = tid < kBN ? kLog2e : 1.0f;
  float val = 0.0f;
  auto fetch = [&](int s) {
    const int h = kvh * prm.G + s / per_head;
    const int qt = qlo + s % per_head;
    const size_t q_slice = (size_t)(b * prm.Hq + h) * N;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(prm.q + q_slice * D, (uint32_t)N * D * 2);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(prm.dout + q_slice * D, (uint32_t)N * D * 2);
    stage.load(rq, ro, qt * kBN, tid);
    const int i = qt * kBN + (tid & (kBN - 1));
    val = row_val && i < N ? val_src[q_slice + i] : 0.0f;
  };
  auto put = [&](lchar *set) {
    stage.template store<st::kB128, st::kTr, true>(set + kQb, set + kQt, set + kOb, set + kOt, tid);
    static_assert(kDel == kLse + 4 * kBN, "lse and Delta arrays must be adjacent");
    if (row_val) ((lds_f32_t *)(set + kLse))[tid] = val * val_mul;
  };

  // edge mask: query row i sees this lane's key iff (unsigned)(i - m_lo) < m_span
  const int m_lo = prm.causal ? key : 0;
  const int m_span = key >= N ? 0
                     : !prm.causal ? N
                     : prm.window > 0 ? min(prm.window, N - key) : N - key;

  // S and dP (32 queries x 32 keys) of row block rb; register r holds query
  // row 32 rb + 8 (r / 4) + 4 hh + r % 4 of the tile
  auto sdp = [&](const lchar *set, int rb, f32x16 &sa, f32x16 &dp) {
    const lchar *qb = set + kQb + qb_lane;
    const lchar *ob = set + kOb + qb_lane;
    sa = f32x16{};
    dp = f32x16{};
#pragma unroll
    for (int kk = 0; kk < st::kKSteps; ++kk) {
      sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b128_frag<st::kB128>(qb, kk, rb), kf[kk], sa, 0,
                                                   0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b128_frag<st::kB128>(ob, kk, rb), vf[kk], dp, 0,
                                                   0, 0);
    }
  };
  // P = exp2(S c - lse log2 e) (zero where masked) and dS = P (dP - Delta),
  // as bf16 B operands
  auto softmax = [&](bool masked, const lchar *set, int q0, int rb, const f32x16 &sa,
                     const f32x16 &dp, bf16x8 (&pf)[2], bf16x8 (&dsf)[2]) {
    const lds_f32x4_t *lsep = (const lds_f32x4_t *)(set + kLse) + 8 * rb + hh;
    const lds_f32x4_t *delp = (const lds_f32x4_t *)(set + kDel) + 8 * rb + hh;
    f32x16 p;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const f32x4 l2 = lsep[2 * a];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        p[4 * a + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[4 * a + e], c, -l2[e]));
    }
    if (masked) {
      const int base = q0 + 32 * rb + 4 * hh - m_lo;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        p[r] = (unsigned)(base + 8 * (r >> 2) + (r & 3)) < (unsigned)m_span ? p[r] : 0.0f;
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const f32x4 dl = delp[2 * a];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * a + e;
        pf[r >> 3][r & 7] = (__bf16)p[r];
        dsf[r >> 3][r & 7] = (__bf16)(p[r] * (dp[r] - dl[e]));
      }
    }
  };
  // dV^T += dO^T P, dK^T += Q^T dS over the 32 rows of block rb
  auto dkdv = [&](const lchar *set, int rb, const bf16x8 (&pf)[2], const bf16x8 (&dsf)[2]) {
    const lchar *qtr = set + kQt + qt_lane;
    const lchar *otr = set + kOt + qt_lane;
#pragma unroll
    for (int db = 0; db < st::kDB; ++db) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        dvacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<st::kTr>(otr, db, rb, tt),
                                                            pf[tt], dvacc[db], 0, 0, 0);
        dkacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<st::kTr>(qtr, db, rb, tt),
                                                            dsf[tt], dkacc[db], 0, 0, 0);
      }
    }
  };
  // One wave per SIMD runs this, so its own instruction order decides how
  // much hides under the matrix cores: the S / dP products of block 1 are
  // issued ahead of the softmax of block 0, and the dV / dK products of
  // block 0 ahead of the softmax of block 1.
  auto tile = [&](bool masked, int q0, const lchar *set) {
    f32x16 s0, d0, s1, d1;
    bf16x8 p0[2], g0[2], p1[2], g1[2];
    sdp(set, 0, s0, d0);
    __builtin_amdgcn_sched_barrier(0);
    sdp(set, 1, s1, d1);
    softmax(masked, set, q0, 0, s0, d0, p0, g0);
    __builtin_amdgcn_sched_barrier(0);
    dkdv(set, 0, p0, g0);
    softmax(masked, set, q0, 1, s1, d1, p1, g1);
    __builtin_amdgcn_sched_barrier(0);
    dkdv(set, 1, p1, g1);
  };
  auto compute = [&](int s, const lchar *set) {
    const int q0 = (qlo + s % per_head) * kBN;  // first query row of the tile
    const bool need_mask = (prm.causal && q0 < kw0 + 31) ||
                           (prm.window > 0 && q0 + kBN - 1 >= kw0 + prm.window) ||
                           (q0 + kBN > N) || (kw0 + 31 >= N);
    tile(need_mask, q0, set);
  };

  lchar *const set0 = (lchar *)smem;
  lchar *const set1 = (lchar *)smem + kSet;
  if (steps > 0) {
    fetch(0);
    put(set0);
  }
  __syncthreads();
  auto step = [&](int s, const lchar *cur, lchar *next) {
    const bool more = s + 1 < steps;
    if (more) fetch(s + 1);
    const int qt = qlo + s % per_head;
    if (qt >= wlo && qt < whi) compute(s, cur);
    if (more) put(next);
    __syncthreads();
  };
  for (int s = 0; s < steps; s += 2) {
    step(s, set0, set1);
    if (s + 1 < steps) step(s + 1, set1, set0);
  }

  if (key < N) {
    store_rows<D>(prm.dk + kv_slice * D, key, hh, dkacc, prm.scale);
    store_rows<D>(prm.dv + kv_slice * D, key, hh, dvacc, 1.0f);
  }
}

template <int D>
BwdParams make_params(const BwdProblem &p) {
  BwdParams prm;
  prm.q = static_cast<const uint16_t *>(p.q);
  prm.k = static_cast<const uint16_t *>(p.k);
  prm.v = static_cast<const uint16_t *>(p.v);
  prm.o = static_cast<const uint16_t *>(p.o);
  prm.dout = static_cast<const uint16_t *>(p.dout);
  prm.lse = p.lse;
  prm.delta = p.delta;
  prm.dq = static_cast<uint16_t *>(p.dq);
  prm.dk = static_cast<uint16_t *>(p.dk);
  prm.dv = static_cast<uint16_t *>(p.dv);
  prm.B = p.B; prm.Hq = p.Hq; prm.Hkv = p.Hkv; prm.N = p.N;
  prm.G = p.Hq / p.Hkv;
  prm.nkt = (p.N + kBN - 1) / kBN;
  prm.c = p.scale * kLog2e;
  prm.scale = p.scale;
  prm.causal = p.causal;
  prm.window = p.window;
  return prm;
}

template <int D, int P>
hipError_t launch_dq(BwdParams prm, hipStream_t stream) {
  constexpr int NW = 8;
  constexpr int kRows = 32 * NW / P;
  prm.groups = prm.Hq / P;
  prm.nq = (prm.N + kRows - 1) / kRows;
  const long long total = (long long)prm.B * prm.groups * prm.nq;
  if (total > 0x7fffffffLL) return hipErrorInvalidValue;
  prm.total = (int)total;
  void *args[] = {&prm};
  return hipLaunchKernel(reinterpret_cast<const void *>(&attn_bwd_dq_kernel<D, NW, P>),
                         dim3(prm.total), dim3(NW * 64), args, 0, stream);
}

template <int D>
hipError_t launch_bwd_d(const BwdProblem &p, hipStream_t stream) {
  BwdParams prm = make_params<D>(p);
  {
    const long long rows = (long long)p.B * p.Hq * p.N;
    const long long blocks = (rows + 63) / 64;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    void *args[] = {&prm};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&attn_bwd_delta_kernel<D>),
                                         dim3((unsigned)blocks), dim3(256), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  {
    const int G = prm.G;
    const hipError_t e = G % 8 == 0   ? launch_dq<D, 8>(prm, stream)
                         : G % 4 == 0 ? launch_dq<D, 4>(prm, stream)
                         : G % 2 == 0 ? launch_dq<D, 2>(prm, stream)
                                      : launch_dq<D, 1>(prm, stream);
    if (e != hipSuccess) return e;
  }
  {
    constexpr int NW = 4;
    prm.nkb = (p.N + 32 * NW - 1) / (32 * NW);
    const long long total = (long long)p.B * p.Hkv * prm.nkb;
    if (total > 0x7fffffffLL) return hipErrorInvalidValue;
    prm.total = (int)total;
    void *args[] = {&prm};
    return hipLaunchKernel(reinterpret_cast<const void *>(&attn_bwd_dkdv_kernel<D, NW>),
                           dim3(prm.total), dim3(NW * 64), args, 0, stream);
  }
}

}  // namespace

hipError_t launch_bwd(const BwdProblem &p, hipStream_t stream) {
  return p.d == 128 ? launch_bwd_d<128>(p, stream) : launch_bwd_d<64>(p, stream);
}

}  // namespace attn
