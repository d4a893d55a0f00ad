// gfx950 (MI355X, CDNA4) exact tiled attention forward.
//
// What is computed: O = softmax(scale * Q K^T) V with masked scores set to
// -inf before the softmax, plus the per-row natural logsumexp of the scaled
// scores ("Efficient Attention: FlashAttention, Sparse, Linear", section
// 45.2.1; "Efficient attention: long context and sub-quadratic variants",
// sections "Sliding-window and local attention" and "Implementation, twice").
// How: the score matrix is produced one 64-key tile at a time on chip and
// folded into a running output with the running (max, sum) softmax of the
// same page's section "FlashAttention: exact attention, IO-aware"; tiles that
// no row can see are never visited ("Against the real libraries": mask
// structure becomes loop bounds).
//
// Mapping onto CDNA4
// ------------------
// * One wave owns 32 query rows of one head.  It computes the transposed
//   score tile S^T = K Q^T (keys x queries) with v_mfma_f32_32x32x16_bf16:
//   A = K rows from LDS, B = Q^T held in registers for the whole kernel.
//   In the 32x32 accumulator, lane l holds query column l % 32 and the keys
//   8*(r/4) + 4*(l/32) + r%4 for r = 0..15, so every softmax row statistic is
//   lane-local up to one exchange between lane l and lane l ^ 32
//   (v_permlane32_swap).
// * The same accumulator registers, rounded to bf16, are directly the B
//   operand of O^T += V^T P^T (a 16-key k-step takes registers 8t..8t+7,
//   i.e. keys 16t + 8*(s/4) + 4*(l/32) + s%4 for slot s), so P never leaves
//   registers.  The matching V^T A operand is read from key-major LDS with
//   ds_read_b64_tr_b16: in each 16-lane group, lane 4j+c supplies the address
//   of 4 consecutive d values of key row j and lane i receives the 4 keys of
//   column i.
// * K and V tiles go HBM -> registers -> LDS, 16 bytes per lane per load.
//   Two register stages keep the next two tiles in flight, so a tile's loads
//   are issued two tiles of MFMAs before their LDS stores.  (Direct buffer_load ... lds would save the registers, but
//   into one LDS array the compiler waits for every outstanding vector load
//   before each LDS read; with one array per buffer it does not, yet a
//   wave's direct load fills 64 consecutive 16-byte slots, which the padded
//   rows below do not form.)  The buffer descriptor spans one (batch, KV-head)
//   slice, so keys past N read as zero.  LDS rows are padded so both the
//   b128 K reads and the transposed V reads hit distinct banks.
// * GQA: the query heads sharing a KV head are packed into one workgroup
//   (one head per wave), so each K/V tile is loaded once for all of them.
// * Online softmax with a lazy reference max: O is rescaled only when a
//   row's tile max exceeds the reference by more than 2^kTau, and O is
//   normalized by the sum of the bf16 weights the MFMA actually used.
//
// Schedule: per key tile, every wave runs S, softmax and PV between two
// workgroup barriers; the two waves that share a SIMD (8-wave variant) run
// their softmax together, which is what keeps the vector ALU busy: one wave
// alone issues a vector instruction only every few clocks.  At d = 64 the
// default is the 4-wave variant: it fits three workgroups per CU, whose
// waves (held together by no barrier) overlap one another's softmax and
// matrix products.

#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "attn_device.h"
#include "attn_internal.h"

namespace attn {
namespace {

using dev::bf16x2;
using dev::bf16x4;
using dev::bf16x8;
using dev::f32x16;
using dev::i16x4;
using dev::kLn2;
using dev::kLog2e;
using dev::lchar;
using dev::lds_bf16x8_t;
using dev::lds_i16x4_t;
using dev::lds_u32x4_t;
using dev::make_rsrc;
using dev::u32x4;
using dev::wave_max_pair;
using dev::wave_sum_pair;
using dev::causal_window_keys;
using dev::dense_slot;
using dev::edge_tile;
using dev::tile_slot;
using dev::TileSlot;

constexpr int kBN = 64;              // keys per tile
constexpr float kTau = 16.0f;        // lazy-rescale threshold, log2 units

struct Params {
  const uint16_t *q, *k, *v;
  uint16_t *o;
  float *lse;
  int B, Hq, Hkv, N;
  int G;          // Hq / Hkv
  int groups;     // Hq / P (head groups, one per workgroup column)
  int nq;         // query tiles per head group
  int total;      // workgroups
  int nkt;        // key tiles = ceil(N / 64)
  float c;        // |scale| * log2(e), at least FLT_MIN
  int neg;        // scale < 0: Q is negated on load, exact in bf16
  int causal;
  int window;     // 0: none
  // packed variable-length batches and local + global masks (GEN kernels
  // only): sequence b is rows cu[b] .. cu[b+1]-1 of every head's
  // [total_rows][D] slice; query and key rows below nglob are global; a
  // radius > 0 limits the others to |i - j| <= radius
  const int *cu;
  int total_rows;
  int radius;
  int nglob;
  int compact;    // sequence lengths differ: launch only non-empty tiles first
  int slots;      // persistent launch: workgroups per XCD (0: one per tile)
  // global rows computed by workgroups of their own (global_rows_task): the
  // first ngtask workgroups of the launch; the others treat global rows as
  // local ones and do not write them
  int gsplit;
  int ngtask;
};

template <int D>
struct Geo {
  static constexpr int kRowB = D * 2;           // bytes per K/V row in HBM
  static constexpr int kCh = kRowB / 16;        // 16-byte chunks per row
  // LDS row strides.  K rows are padded by 16 bytes, so the 16 rows one
  // ds_read_b128 phase touches start 4 banks apart; V rows by 64 bytes, so
  // the 4 consecutive rows of a transposed read start 16 banks apart.  Every
  // fragment address is then a per-lane base plus a compile-time offset.
  static constexpr int kKStride = kRowB + 16;
  static constexpr int kVStride = kRowB + 64;
  static constexpr int kKTileB = kBN * kKStride;
  static constexpr int kVTileB = kBN * kVStride;
  static constexpr int kSetB = kKTileB + kVTileB;  // one K tile + one V tile
  static constexpr int kKSteps = D / 16;        // MFMA k-steps of S^T
  static constexpr int kDB = D / 32;            // 32-wide d blocks of O^T
  static constexpr int kS = 2 * kKSteps;        // S MFMAs per tile
  static constexpr int kPV = 4 * kDB;           // PV MFMAs per tile
};


// This thread's share of one K tile and one V tile (possibly of different
// key tiles): kLoads 16-byte chunks each.  Chunk n covers tile row
// r = ci / kCh, chunk p = ci % kCh with ci = n * NW * 64 + tid, so each wave
// instruction reads whole rows contiguously from HBM.  Keys past N read as
// zero (buffer range check).
template <int D, int NW>
struct TileStage {
  using g = Geo<D>;
  static constexpr int kLoads = kBN * g::kCh / (NW * 64);
  static_assert(kLoads * NW * 64 == kBN * g::kCh, "tile must split evenly over the threads");
  u32x4 k[kLoads], v[kLoads];

  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                       int jk0, int jv0, int tid) {
#pragma unroll
    for (int n = 0; n < kLoads; ++n) {
      const int ci = n * NW * 64 + tid;
      k[n] = __builtin_amdgcn_raw_buffer_load_b128(rk, jk0 * g::kRowB + ci * 16, 0, 0);
      v[n] = __builtin_amdgcn_raw_buffer_load_b128(rv, jv0 * g::kRowB + ci * 16, 0, 0);
    }
  }
  // Write the K chunks into the K tile at `kt` and the V chunks into the V
  // tile at `vt`, each row at its padded stride.
  __device__ __forceinline__ void store(lchar *kt, lchar *vt, int tid) const {
    const int r0 = tid / g::kCh, p = tid % g::kCh;
    lchar *kp = kt + r0 * g::kKStride + p * 16;
    lchar *vp = vt + r0 * g::kVStride + p * 16;
    constexpr int kRowsPerLoad = NW * 64 / g::kCh;
#pragma unroll
    for (int n = 0; n < kLoads; ++n) {
      *(lds_u32x4_t *)(kp + n * kRowsPerLoad * g::kKStride) = k[n];
      *(lds_u32x4_t *)(vp + n * kRowsPerLoad * g::kVStride) = v[n];
    }
  }
};


// The key tiles a block of query rows visits: [0, a_hi) then [b_lo, b_hi)
// (disjoint, a_hi < b_lo).  The first range holds the global keys, the
// second the causal / window / radius band; a block holding a global row
// visits every key it may see.  Without global tokens it is one range.
struct Segs {
  int a_hi, b_lo, b_hi;
  __device__ __forceinline__ int count() const { return a_hi + max(b_hi - b_lo, 0); }
  __device__ __forceinline__ int tile(int k) const { return k < a_hi ? k : b_lo + (k - a_hi); }
  __device__ __forceinline__ bool has(int t) const { return t < a_hi || (t >= b_lo && t < b_hi); }
};

// Rows [r0, r1) of a sequence of N rows (r0 < r1 <= N).
__device__ __forceinline__ Segs key_segments(const Params &prm, int r0, int r1, int N) {
  int lo, hi;
  causal_window_keys(prm.causal, prm.window, r0, r1, N, lo, hi);
  const int hi_c = hi;  // keys past this are never seen
  Segs sg;
  if (r0 < prm.nglob && !prm.gsplit) {  // a global row sees every key it may
    sg.a_hi = 0;
    sg.b_lo = 0;
    sg.b_hi = (hi_c + kBN - 1) / kBN;
    return sg;
  }
  if (prm.radius > 0) {
    lo = max(lo, r0 - prm.radius);
    hi = min(hi, r1 + prm.radius);
  }
  sg.a_hi = (min(prm.nglob, hi_c) + kBN - 1) / kBN;
  sg.b_lo = lo / kBN;
  sg.b_hi = (hi + kBN - 1) / kBN;
  if (sg.b_lo <= sg.a_hi) {  // the ranges touch: one range
    sg.a_hi = max(sg.a_hi, sg.b_hi);
    sg.b_lo = sg.b_hi = sg.a_hi;
  }
  return sg;
}

// Which (batch, head, rows, key tiles) a wave of a workgroup owns.
struct Task {
  int b, head, kvh;
  int N;               // rows of this sequence
  int qw0;             // first query row of this wave
  Segs wg;             // key tiles any row of the workgroup sees
  Segs w;              // key tiles any row of this wave sees
  size_t q_slice;      // first row of the Q / O slice
  size_t kv_slice;     // first row of the K / V slice
  bool empty;          // no row of the workgroup lies inside its sequence
};

// Sum over the wave, returned as a scalar (so everything derived from it
// stays in scalar registers).
__device__ __forceinline__ int wave_sum_int(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return __builtin_amdgcn_readfirstlane(x);
}

// Packed sequences of different lengths leave many (rank, sequence) slots
// of the rank-major order empty: a short sequence has no tile at the high
// ranks.  Scattered through the launch order, such workgroups cost almost
// as much as short real ones.  Compacted order: workgroup n takes the n-th
// non-empty (rank, sequence, head group) in the same rank-major order, so
// the empty ones all come last.  S(r) = number of non-empty (rank, sequence)
// slots below rank r; workgroup n serves slot m = n / groups at the largest
// r with S(r) <= m.  Each wave computes it with its lanes over the
// sequences (all wave-uniform results).  Returns false past the last slot.
template <int kRows>
__device__ __forceinline__ bool compact_slot(const Params &prm, int n, int &rank, int &b_out,
                                             int &hg) {
  const int lane = threadIdx.x & 63;
  const int nq = prm.nq;
  auto tiles_of = [&](int b) {  // row tiles of sequence b (0 past the end)
    if (b >= prm.B) return 0;
    const int s0 = min(max(prm.cu[b], 0), prm.total_rows);
    const int s1 = min(max(prm.cu[b + 1], 0), prm.total_rows);
    return min((max(s1 - s0, 0) + kRows - 1) / kRows, nq);  // rows past nq * kRows: no tile
  };
  // slots of one sequence below rank r: causal ranks run heaviest (last)
  // row tile first, so sequence b first appears at rank nq - nt
  auto below = [&](int nt, int r) { return prm.causal ? max(0, r - (nq - nt)) : min(r, nt); };
  const int nt0 = tiles_of(lane);
  const int nchunks = (prm.B + 63) / 64;
  auto S = [&](int r) {
    int acc = below(nt0, r);
    for (int c = 1; c < nchunks; ++c) acc += below(tiles_of(64 * c + lane), r);
    return wave_sum_int(acc);
  };
  const int m = n / prm.groups;
  hg = n % prm.groups;
  int lo = 0, hi = nq;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (S(mid) <= m) lo = mid; else hi = mid - 1;
  }
  if (lo >= nq) return false;
  rank = lo;
  const int qi = prm.causal ? nq - 1 - lo : lo;
  int jb = m - S(lo);  // the jb-th sequence (in batch order) with a tile at this rank
  for (int c = 0; c < nchunks; ++c) {
    const int nt = c == 0 ? nt0 : tiles_of(64 * c + lane);
    const unsigned long long has = __builtin_amdgcn_ballot_w64(qi < nt);
    const int cnt = __popcll(has);
    if (jb < cnt) {
      const int before = __popcll(has & ((1ull << lane) - 1ull));
      const unsigned long long pick = __builtin_amdgcn_ballot_w64(qi < nt && before == jb);
      b_out = 64 * c + __ffsll((long long)pick) - 1;
      return true;
    }
    jb -= cnt;
  }
  return false;
}

// kRows query rows per workgroup, P heads per workgroup (wave w serves head
// w % P on rows (w / P) * 32 ..).  GEN: packed sequences [cu[b], cu[b+1]).
template <int P, int kRows, bool GEN>
__device__ __forceinline__ Task make_task(const Params &prm, int wave, int pq = -1, int phgb = -1) {
  Task tk;
  int qrank, hgb;
  if (!GEN && pq >= 0) {  // given by the persistent schedule
    qrank = pq;
    hgb = phgb;
  } else if constexpr (GEN) {
    // packed sequences of different lengths: tile rank slowest, so the
    // heaviest tiles of every sequence go first and consecutive workgroups
    // (dealt round-robin to the XCDs) spread every sequence over all XCDs
    if (prm.compact) {
      int b, hg;
      if (!compact_slot<kRows>(prm, (int)blockIdx.x - prm.ngtask, qrank, b, hg)) {
        tk.empty = true;
        return tk;
      }
      hgb = b * prm.groups + hg;
    } else {
      const int nbh = prm.B * prm.groups;
      const int id = (int)blockIdx.x - prm.ngtask;
      qrank = id / nbh;
      hgb = id % nbh;
    }
  } else {
    dense_slot(prm, blockIdx.x, qrank, hgb);
  }
  const TileSlot sl = tile_slot<P, kRows>(prm, wave, qrank, hgb);
  tk.b = sl.b;
  tk.head = sl.head;
  tk.kvh = sl.kvh;
  tk.qw0 = sl.qw0;
  const int wg_r0 = sl.wg_r0;
  int N;
  if constexpr (GEN) {
    // offsets clamped into [0, total_rows]: an inconsistent table yields
    // empty or shortened sequences, never reads outside the tensors
    const int start = min(max(prm.cu[tk.b], 0), prm.total_rows);
    N = min(prm.cu[tk.b + 1], prm.total_rows) - start;
    tk.kv_slice = (size_t)tk.kvh * prm.total_rows + start;
    tk.q_slice = (size_t)tk.head * prm.total_rows + start;
  } else {
    N = prm.N;
    tk.kv_slice = (size_t)(tk.b * prm.Hkv + tk.kvh) * N;
    tk.q_slice = (size_t)(tk.b * prm.Hq + tk.head) * N;
  }
  tk.N = N;
  tk.empty = wg_r0 >= N;
  if (tk.empty) return tk;
  tk.wg = key_segments(prm, wg_r0, min(N, wg_r0 + kRows), N);
  if (tk.qw0 < N) {
    tk.w = key_segments(prm, tk.qw0, min(N, tk.qw0 + 32), N);
  } else {
    tk.w = Segs{0, 0, 0};  // rows past the end: this wave only helps load tiles
  }
  return tk;
}

// Q^T operand: lane holds query row qw0 + l32, d = 16*kk + 8*hh + s.
template <int D>
__device__ __forceinline__ void load_q(const Params &prm, const Task &tk, int l32, int hh,
                                       bf16x8 (&qf)[Geo<D>::kKSteps]) {
  const int row = tk.qw0 + l32;
  const uint16_t *qp = prm.q + tk.q_slice * D + (size_t)row * D + 8 * hh;
#pragma unroll
  for (int kk = 0; kk < Geo<D>::kKSteps; ++kk) {
    qf[kk] = row < tk.N ? *(const bf16x8 *)(qp + 16 * kk) : bf16x8{};
    if (prm.neg) {
      u32x4 t = __builtin_bit_cast(u32x4, qf[kk]);
      t ^= 0x80008000u;
      qf[kk] = __builtin_bit_cast(bf16x8, t);
    }
  }
}

// Per-lane LDS byte offsets of the MFMA fragments.
// K (b128): key row 32*rb + l32, d = 16*kk + 8*hh .. +7.
template <int D>
__device__ __forceinline__ int k_lane_off(int lane) {
  return (lane & 31) * Geo<D>::kKStride + (lane >> 5) * 16;
}
// V (transposed read): key row 32rb + 16tt + 8u + 4hh + (lane & 15) / 4,
// d = 32db + 16*((lane >> 4) & 1) + 4*(lane & 3) .. +3.
template <int D>
__device__ __forceinline__ int v_lane_off(int lane) {
  return (4 * (lane >> 5) + ((lane & 15) >> 2)) * Geo<D>::kVStride +
         (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
}
// K fragment (k-step kk, key block rb) from a K tile base already offset by
// k_lane_off.
template <int D>
__device__ __forceinline__ bf16x8 kfrag(const lchar *kb, int kk, int rb) {
  return *(const lds_bf16x8_t *)(kb + rb * 32 * Geo<D>::kKStride + kk * 32);
}
// V^T fragment (d block db, key block rb, 16-key half tt) from a V tile base
// already offset by v_lane_off: two transposed reads of 4 keys each.
template <int D>
__device__ __forceinline__ bf16x8 vfrag(const lchar *vb, int db, int rb, int tt) {
  const lchar *p = vb + (32 * rb + 16 * tt) * Geo<D>::kVStride + db * 64;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)p);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(p + 8 * Geo<D>::kVStride));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, both);
}

// Running softmax state of the lane's query row (its half of the keys).
struct RowState {
  float m2 = -1e30f;   // reference max, scaled log2 units (finite: no inf - inf)
  float lsum = 0.0f;   // sum of the fp32 weights (gives lse)
  float lrnd = 0.0f;   // sum of the bf16-rounded weights (normalizes O)
};

// Whether key tile j0 holds a (row, key) pair that a row of the wave's 32
// rows qw0.. cannot see: the causal diagonal, the window edge and the tile
// holding key N - 1.  Wave-uniform.
__device__ __forceinline__ bool tile_needs_mask(const Params &prm, int j0, int qw0, int N) {
  return edge_tile(prm.causal, prm.window, j0, kBN, qw0, N);
}

// Scores of keys this lane's row cannot see become -inf.  SPLIT (the
// ping-pong kernel): tiles with no window edge take one signed compare per
// score, the others the range compare; the lockstep kernels keep the single
// range compare (a second code path there cost registers and spills).
template <bool SPLIT>
__device__ __forceinline__ void apply_mask(f32x16 (&s)[2], const Params &prm, int j0, int qw0,
                                           int l32, int hh, int N) {
  // Register r of block rb holds key kbase + off with the compile-time
  // off = 32*rb + 8*(r/4) + r%4.  The keys this lane's row sees form the
  // range lo < off <= hi relative to kbase, so one unsigned compare per
  // register decides visibility: (unsigned)(off - lo - 1) < hi - lo.
  const int qrow = qw0 + l32;
  const int kbase = j0 + 4 * hh;
  int hi = N - 1 - kbase;
  if (prm.causal) hi = min(hi, qrow - kbase);
  if (!SPLIT || (prm.window > 0 && j0 <= qw0 + 31 - prm.window)) {  // a lower edge too
    const int lo = prm.window > 0 ? qrow - prm.window - kbase : -1 - kbase;
    const unsigned span = (unsigned)max(hi - lo, 0);
    const int lo1 = lo + 1;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 32 * rb + 8 * (r >> 2) + (r & 3);
        const bool vis = (unsigned)(off - lo1) < span;
        s[rb][r] = vis ? s[rb][r] : -INFINITY;
      }
    }
  } else {  // only an upper edge (the diagonal, N): one signed compare per score
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 32 * rb + 8 * (r >> 2) + (r & 3);
        s[rb][r] = off <= hi ? s[rb][r] : -INFINITY;
      }
    }
  }
}

// The general rule of the GEN kernels: row i sees key j < N iff
//   (not causal or j <= i) and (i < nglob or j < nglob or
//    ((window <= 0 or j > i - window) and (radius <= 0 or |i - j| <= radius))).
__device__ __forceinline__ bool tile_needs_mask_gen(const Params &prm, int j0, int qw0, int N) {
  if (j0 + kBN > N || (prm.causal && j0 + kBN - 1 > qw0)) return true;
  if ((qw0 + 31 < prm.nglob && !prm.gsplit) || j0 + kBN - 1 < prm.nglob) return false;
  const bool win_ok = prm.window <= 0 || j0 > qw0 + 31 - prm.window;
  const bool rad_ok = prm.radius <= 0 ||
                      (j0 >= qw0 + 31 - prm.radius && j0 + kBN - 1 <= qw0 + prm.radius);
  return !(win_ok && rad_ok);
}

// The keys row i sees are two ranges: the global keys [0, gcap) and the
// local range [lo, hi] (for a global row: every key it may see).  With the
// per-register offset off (key = kbase + off), each is one unsigned compare.
// SPLIT (the ping-pong kernel): a tile with no global key takes the local
// range compare alone (the lockstep kernels' register budget has no room for
// the second code path).
template <bool SPLIT>
__device__ __forceinline__ void apply_mask_gen(f32x16 (&s)[2], const Params &prm, int j0,
                                               int qw0, int l32, int hh, int N) {
  const int i = qw0 + l32;
  const int hi_c = prm.causal ? min(i, N - 1) : N - 1;  // last key causality allows
  int lo = 0, hi = hi_c;
  if (i >= prm.nglob || prm.gsplit) {
    if (prm.window > 0) lo = max(lo, i - prm.window + 1);
    if (prm.radius > 0) {
      lo = max(lo, i - prm.radius);
      hi = min(hi, i + prm.radius);
    }
  }
  const int gcap = min(prm.nglob, hi_c + 1);
  const int kbase = j0 + 4 * hh;
  const int a = kbase - lo;                       // key - lo = off + a
  const unsigned span = (unsigned)max(hi - lo + 1, 0);
  if (SPLIT && j0 >= prm.nglob) {  // no global key in the tile: the local range alone
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 32 * rb + 8 * (r >> 2) + (r & 3);
        s[rb][r] = (unsigned)(off + a) < span ? s[rb][r] : -INFINITY;
      }
    }
    return;
  }
  const unsigned gspan = (unsigned)max(gcap, 0);  // key < gcap
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int off = 32 * rb + 8 * (r >> 2) + (r & 3);
      const bool vis = (unsigned)(off + a) < span || (unsigned)(off + kbase) < gspan;
      s[rb][r] = vis ? s[rb][r] : -INFINITY;
    }
  }
}

template <bool GEN, bool SPLIT = false>
__device__ __forceinline__ void mask_tile(f32x16 (&s)[2], const Params &prm, int j0, int qw0,
                                          int l32, int hh, int N) {
  if constexpr (GEN) {
    if (tile_needs_mask_gen(prm, j0, qw0, N)) apply_mask_gen<SPLIT>(s, prm, j0, qw0, l32, hh, N);
  } else {
    if (tile_needs_mask(prm, j0, qw0, N)) apply_mask<SPLIT>(s, prm, j0, qw0, l32, hh, N);
  }
}

// Online softmax of one tile of scores (scaled log2 domain), without
// branches: new tile max; lazy move of the reference max m2 (it moves only
// when some row's tile max exceeds it by more than kTau log2 units, so
// P <= 2^kTau, and then every row of the wave takes its exact running max);
// P = exp2(c*S - m2) packed to bf16 as the B operand of the PV MFMAs; both
// running sums.  Returns whether m2 moved; the caller then multiplies O by
// `alpha` before the next PV MFMA.
// NB: key blocks of 32 in the tile (2; 1 for the 32-key tiles of the global
// rows, whose second block is unused).
template <int NB = 2>
__device__ __forceinline__ bool softmax_core(const f32x16 (&s)[2], bf16x8 (&pf)[2][2],
                                             RowState &st, float c, float &alpha) {
  float mq[4];  // independent max chains, two per block
#pragma unroll
  for (int j = 0; j < 2 * NB; ++j) mq[j] = fmaxf(s[j >> 1][8 * (j & 1)], s[j >> 1][8 * (j & 1) + 1]);
#pragma unroll
  for (int j = 0; j < 2 * NB; ++j) {
#pragma unroll
    for (int e = 2; e < 8; ++e) mq[j] = fmaxf(mq[j], s[j >> 1][8 * (j & 1) + e]);
  }
  if constexpr (NB == 1) {
    mq[2] = mq[0];
    mq[3] = mq[1];
  }
  const float mx = wave_max_pair(fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3])));
  const float mt2 = mx * c;
  const bool move = __builtin_amdgcn_ballot_w64(mt2 > st.m2 + kTau) != 0;
  const float mnew = move ? fmaxf(st.m2, mt2) : st.m2;
  alpha = __builtin_amdgcn_exp2f(st.m2 - mnew);
  st.lsum *= alpha;
  st.lrnd *= alpha;
  st.m2 = mnew;
  const float negm = -st.m2;
  float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // independent add chains
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rb][8 * tt + e], c, negm));
        part[e & 3] += p;
        pf[rb][tt][e] = (__bf16)p;
      }
    }
  }
  st.lsum += (part[0] + part[1]) + (part[2] + part[3]);
  // The same weights as the PV MFMA sees them (bf16), summed with
  // v_dot2_f32_bf16 against (1, 1): normalizing O by this sum makes a row
  // dominated by one key return that key's V row up to fp32 rounding, even
  // when its weight is not exactly 1.0 (lazy rescale).
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float rp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16x2 pair = {pf[rb][tt][2 * e], pf[rb][tt][2 * e + 1]};
        rp[e] = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, rp[e], false);
      }
    }
  }
  st.lrnd += (rp[0] + rp[1]) + (rp[2] + rp[3]);
  return move;
}

template <int KDB, int NB = 2>
__device__ __forceinline__ void softmax_tile(const f32x16 (&s)[2], bf16x8 (&pf)[2][2],
                                             RowState &st, f32x16 (&oacc)[KDB], float c) {
  float alpha;
  if (softmax_core<NB>(s, pf, st, c, alpha)) {
#pragma unroll
    for (int i = 0; i < KDB; ++i) oacc[i] *= alpha;
  }
}

// Epilogue: O = O / lrnd (bf16, RNE) and lse = ln(lsum) + max, for rows
// row_lo .. N - 1 (rows below row_lo belong to global_rows_task).
template <int D>
__device__ __forceinline__ void write_out(const Params &prm, const Task &tk, int l32, int hh,
                                          const f32x16 (&oacc)[Geo<D>::kDB], const RowState &st,
                                          int row_lo = 0) {
  const float ltot = wave_sum_pair(st.lsum);
  const float lrtot = wave_sum_pair(st.lrnd);
  const int row = tk.qw0 + l32;
  if (row >= tk.N || row < row_lo) return;
  const float inv = 1.0f / lrtot;
  uint16_t *op = prm.o + tk.q_slice * D + (size_t)row * D + 4 * hh;
#pragma unroll
  for (int db = 0; db < Geo<D>::kDB; ++db) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = (__bf16)(oacc[db][4 * i + j] * inv);
      *(bf16x4 *)(op + 32 * db + 8 * i) = w;
    }
  }
  if (hh == 0) prm.lse[tk.q_slice + row] = (st.m2 + __builtin_amdgcn_logf(ltot)) * kLn2;
}

// ---------------------------------------------------------------------------
// Global rows (Longformer's global tokens, general mode).  A global row sees
// every key, so the workgroup holding one would run the whole key range
// while the others run their band: it would set the end of the launch.
// Instead the first ngtask workgroups of the launch each take one block of
// 32 global rows of one (sequence, query head) and split its keys over four
// waves: wave w runs the 32-key tiles w, w + 4, ... on its own LDS quarter
// (one wave's LDS instructions run in order, so no barrier is needed
// between a tile's reads and the next tile's stores), with the forward's
// arithmetic (lazy reference max, P in bf16, both sums).  The four partial
// states (m, l, l~, O) are then merged through LDS by the rule the running
// softmax uses: M = max_w m_w, each part weighted by 2^(m_w - M).  The
// other workgroups treat the global rows as local ones and do not write
// them.
// ---------------------------------------------------------------------------
template <int D>
struct HalfTile {  // 32 keys of K and V in registers: 16-byte chunks per lane
  using g = Geo<D>;
  static constexpr int kN = 32 * g::kCh / 64;  // chunks per lane per tensor
  u32x4 k[kN], v[kN];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                       int j0, int lane) {
#pragma unroll
    for (int n = 0; n < kN; ++n) {
      const int ci = n * 64 + lane, r = ci / g::kCh, c = ci % g::kCh;
      const uint32_t off = (uint32_t)(j0 + r) * g::kRowB + c * 16;
      k[n] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
      v[n] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
    }
  }
  __device__ __forceinline__ void store(lchar *kt, lchar *vt, int lane) const {
#pragma unroll
    for (int n = 0; n < kN; ++n) {
      const int ci = n * 64 + lane, r = ci / g::kCh, c = ci % g::kCh;
      *(lds_u32x4_t *)(kt + r * g::kKStride + c * 16) = k[n];
      *(lds_u32x4_t *)(vt + r * g::kVStride + c * 16) = v[n];
    }
  }
};

template <int D>
__device__ __forceinline__ void global_rows_task(const Params &prm, char *smem) {
  using g = Geo<D>;
  constexpr int kW = 4;                          // waves that split the keys
  constexpr int kQuarterB = g::kSetB / 2;        // 32-key K tile + 32-key V tile
  constexpr int kVOff = 32 * g::kKStride;
  static_assert(kW * kQuarterB <= 2 * g::kSetB, "four quarters in the two buffer sets");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;

  const int ngb = (prm.nglob + 31) / 32;
  const int gb = (int)blockIdx.x % ngb, bh = (int)blockIdx.x / ngb;
  const int h = bh % prm.Hq, b = bh / prm.Hq;
  const int start = min(max(prm.cu[b], 0), prm.total_rows);
  const int N = max(min(prm.cu[b + 1], prm.total_rows) - start, 0);
  const int nrows = min(prm.nglob, N);  // global rows of this sequence
  Task tk;
  tk.b = b;
  tk.head = h;
  tk.kvh = h / prm.G;
  tk.N = N;
  tk.qw0 = 32 * gb;
  tk.q_slice = (size_t)h * prm.total_rows + start;
  tk.kv_slice = (size_t)tk.kvh * prm.total_rows + start;
  if (tk.qw0 >= nrows) return;  // the whole workgroup

  f32x16 oacc[g::kDB];
#pragma unroll
  for (int i = 0; i < g::kDB; ++i) oacc[i] = f32x16{};
  RowState st;
  const float c = prm.c;
  if (wave < kW) {
    bf16x8 qf[g::kKSteps];
    load_q<D>(prm, tk, l32, hh, qf);
#pragma unroll
    for (int kk = 0; kk < g::kKSteps; ++kk) asm volatile("" : "+v"(qf[kk]) : : "memory");
    lchar *const kt = (lchar *)smem + wave * kQuarterB;
    lchar *const vt = kt + kVOff;
    const __amdgpu_buffer_rsrc_t rs_k = make_rsrc(prm.k + tk.kv_slice * D, (uint32_t)N * D * 2);
    const __amdgpu_buffer_rsrc_t rs_v = make_rsrc(prm.v + tk.kv_slice * D, (uint32_t)N * D * 2);
    const int row = tk.qw0 + l32;
    const int kend = prm.causal ? min(N, tk.qw0 + 32) : N;  // keys any row of the block sees
    const int nt = (kend + 31) / 32;
    const lchar *kb = kt + k_lane_off<D>(lane);
    const lchar *vb = vt + v_lane_off<D>(lane);
    // S^T of 32-key tile j from the wave's LDS quarter, mask, softmax, PV
    auto compute = [&](int j) {
      f32x16 sc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int kk = 0; kk < g::kKSteps; ++kk)
        sc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag<D>(kb, kk, 0), qf[kk], sc[0], 0, 0, 0);
      // register r holds key 32 j + 8 (r / 4) + 4 hh + r % 4; a global row
      // sees every key below N (and, causal, up to itself)
      const int j0 = 32 * j;
      if (j0 + 31 >= N || (prm.causal && j0 + 31 > tk.qw0)) {
        const int hi = (prm.causal ? min(row, N - 1) : N - 1) - (j0 + 4 * hh);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sc[0][r] = 8 * (r >> 2) + (r & 3) <= hi ? sc[0][r] : -INFINITY;
      }
      bf16x8 pf[2][2];
      softmax_tile<g::kDB, 1>(sc, pf, st, oacc, c);  // one block of 32 keys
#pragma unroll
      for (int db = 0; db < g::kDB; ++db) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfrag<D>(vb, db, 0, tt), pf[0][tt],
                                                             oacc[db], 0, 0, 0);
      }
    };
    // tiles j = wave, wave + 4, ...: staged through registers, the next
    // one loading while this one is computed (a second stage would not fit
    // the d = 64 kernel's register budget of three workgroups per CU)
    HalfTile<D> sa;
    if (wave < nt) sa.load(rs_k, rs_v, 32 * wave, lane);
    for (int j = wave; j < nt; j += kW) {
      sa.store(kt, vt, lane);
      if (j + kW < nt) sa.load(rs_k, rs_v, 32 * (j + kW), lane);
      compute(j);
    }
  }
  __syncthreads();  // every wave's tile reads are done: the LDS takes the partial states
  // per wave: m, l, l~ (64 lanes each), then O^T in accumulator order
  constexpr int kStateF = 3 * 64 + g::kDB * 16 * 64;
  static_assert(kW * kStateF * 4 <= 2 * g::kSetB, "partial states fit the LDS");
  float *const part = (float *)smem;
  if (wave < kW) {
    float *const mine = part + wave * kStateF;
    mine[lane] = st.m2;
    mine[64 + lane] = st.lsum;
    mine[128 + lane] = st.lrnd;
#pragma unroll
    for (int db = 0; db < g::kDB; ++db) {
#pragma unroll
      for (int r = 0; r < 16; ++r) mine[192 + (db * 16 + r) * 64 + lane] = oacc[db][r];
    }
  }
  __syncthreads();
  if (wave != 0) return;
  float mx = part[lane];
#pragma unroll
  for (int w = 1; w < kW; ++w) mx = fmaxf(mx, part[w * kStateF + lane]);
  RowState tot;
  tot.m2 = mx;
  tot.lsum = 0.0f;
  tot.lrnd = 0.0f;
#pragma unroll
  for (int db = 0; db < g::kDB; ++db) oacc[db] = f32x16{};
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    const float *const pw = part + w * kStateF;
    const float e = __builtin_amdgcn_exp2f(pw[lane] - mx);  // 0 for a part with no key
    tot.lsum += e * pw[64 + lane];
    tot.lrnd += e * pw[128 + lane];
#pragma unroll
    for (int db = 0; db < g::kDB; ++db) {
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] += e * pw[192 + (db * 16 + r) * 64 + lane];
    }
  }
  Task out = tk;
  out.N = nrows;  // write the global rows only
  write_out<D>(prm, out, l32, hh, oacc, tot);
}

// ---------------------------------------------------------------------------
// Lockstep schedule: per key tile, every wave computes S, softmax and PV
// between two workgroup barriers.
// ---------------------------------------------------------------------------
template <int D, int NW, int P, bool GEN>
__global__ __launch_bounds__(NW * 64, (NW == 4 && D == 64) ? 3 : 2) void attn_fwd_kernel(Params prm) {
  using g = Geo<D>;
  constexpr int kRows = 32 * NW / P;  // query rows per workgroup

  // Two LDS buffer sets, each a K tile followed by a V tile.
  __shared__ __attribute__((aligned(1024))) char smem[2 * g::kSetB];
  lchar *const set0 = (lchar *)smem;
  lchar *const set1 = (lchar *)smem + g::kSetB;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;

  if constexpr (GEN) {
    if ((int)blockIdx.x < prm.ngtask) {
      global_rows_task<D>(prm, smem);
      return;
    }
  }
  const Task tk = make_task<P, kRows, GEN>(prm, wave);
  if (tk.empty) return;  // the whole workgroup: its tile lies past its sequence
  const int N = tk.N;
  const __amdgpu_buffer_rsrc_t rs_k = make_rsrc(prm.k + tk.kv_slice * D, (uint32_t)N * D * 2);
  const __amdgpu_buffer_rsrc_t rs_v = make_rsrc(prm.v + tk.kv_slice * D, (uint32_t)N * D * 2);

  bf16x8 qf[g::kKSteps];
  load_q<D>(prm, tk, l32, hh, qf);
  const int k_lane = k_lane_off<D>(lane);
  const int v_lane = v_lane_off<D>(lane);

  f32x16 oacc[g::kDB];
#pragma unroll
  for (int i = 0; i < g::kDB; ++i) oacc[i] = f32x16{};
  RowState st;
  const float c = prm.c;

  // Q is settled in registers before any tile load is issued, so that no
  // later use of Q waits for the tile loads in flight.
#pragma unroll
  for (int kk = 0; kk < g::kKSteps; ++kk) asm volatile("" : "+v"(qf[kk]) : : "memory");

  // Two register stages: tiles k + 1 and k + 2 are in flight while tile k
  // is computed, so each tile's loads have two tiles of compute to land.
  // Every step issues its loads, past the last tile at row N (outside the
  // buffer range: no memory access, zeros), so the number of loads in
  // flight is the same on every path and each store waits only for its own.
  const int count = tk.wg.count();
  auto row_of = [&](int k) { return k < count ? tk.wg.tile(k) * kBN : N; };
  TileStage<D, NW> stage0, stage1;
  stage0.load(rs_k, rs_v, row_of(0), row_of(0), tid);
  if (count > 0) stage0.store(set0, set0 + g::kKTileB, tid);
  stage1.load(rs_k, rs_v, row_of(1), row_of(1), tid);
  stage0.load(rs_k, rs_v, row_of(2), row_of(2), tid);
  __syncthreads();

  // S^T, mask, online softmax and O^T update for key tile t held in `set`.
  auto compute = [&](const int t, const lchar *const set) {
    const lchar *kb = set + k_lane;
    const lchar *vb = set + g::kKTileB + v_lane;
    constexpr int kKA = 3;  // K ring depth (k-steps in flight)
    constexpr int kVA = 4;  // V ring depth (MFMAs in flight)

    // ---- S^T = K Q^T for 64 keys x 32 queries; K reads run kKA-1 k-steps
    // ahead of the MFMAs that consume them (sched_barrier fences keep the
    // compiler from sinking each read onto its MFMA, which would expose the
    // full LDS latency on every MFMA).
    f32x16 s[2] = {f32x16{}, f32x16{}};
    bf16x8 ka[kKA][2];
#pragma unroll
    for (int kk = 0; kk < kKA - 1; ++kk) {
      ka[kk][0] = kfrag<D>(kb, kk, 0);
      ka[kk][1] = kfrag<D>(kb, kk, 1);
    }
#pragma unroll
    for (int kk = 0; kk < g::kKSteps; ++kk) {
      if (kk + kKA - 1 < g::kKSteps) {
        ka[(kk + kKA - 1) % kKA][0] = kfrag<D>(kb, kk + kKA - 1, 0);
        ka[(kk + kKA - 1) % kKA][1] = kfrag<D>(kb, kk + kKA - 1, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk % kKA][0], qf[kk], s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk % kKA][1], qf[kk], s[1], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // The V^T fragment sequence of the PV MFMAs: i -> (db, rb, tt) =
    // (i / 4, (i / 2) % 2, i % 2).  The first ones do not depend on P:
    // start them now so the softmax hides their latency.
    auto vf = [&](int i) { return vfrag<D>(vb, i >> 2, (i >> 1) & 1, i & 1); };
    bf16x8 va[kVA];
#pragma unroll
    for (int i = 0; i < kVA; ++i) va[i] = vf(i);
    __builtin_amdgcn_sched_barrier(0);

    mask_tile<GEN>(s, prm, t * kBN, tk.qw0, l32, hh, N);
    bf16x8 pf[2][2];
    softmax_tile<g::kDB>(s, pf, st, oacc, c);

    // ---- O^T += V^T P^T; V reads run kVA MFMAs ahead
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < g::kPV; ++i) {
      const int db = i >> 2, rb = (i >> 1) & 1, tt = i & 1;
      const bf16x8 a = va[i % kVA];
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[rb][tt], oacc[db], 0, 0, 0);
      if (i + kVA < g::kPV) va[i % kVA] = vf(i + kVA);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // One key tile: compute it from LDS (if this wave sees any of its keys),
  // park tile k + 1 (loaded two steps earlier) in the other buffer set, and
  // start loading tile k + 3 into the registers that held it.
  auto step = [&](const int k, lchar *const cur_set, lchar *const next_set,
                  TileStage<D, NW> &nxt) {
    const int t = tk.wg.tile(k);
    if (tk.w.has(t)) compute(t, cur_set);
    if (k + 1 < count) nxt.store(next_set, next_set + g::kKTileB, tid);
    nxt.load(rs_k, rs_v, row_of(k + 3), row_of(k + 3), tid);
    __syncthreads();
  };

  // Pairs of steps with no exit between them, so the loads in flight at
  // the loop head are always stage1's then stage0's; an odd last tile runs
  // after the loop.
  int k = 0;
  for (; k + 1 < count; k += 2) {
    step(k, set0, set1, stage1);
    step(k + 1, set1, set0, stage0);
  }
  if (k < count) step(k, set0, set1, stage1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load left in flight

  write_out<D>(prm, tk, l32, hh, oacc, st, prm.gsplit ? prm.nglob : 0);
}

// ---------------------------------------------------------------------------
// Ping-pong schedule (8 waves).  The two waves that share a SIMD belong to
// different groups: A = waves 0-3, B = waves 4-7.  The workgroup advances in
// half-steps separated by barriers; in every half-step one group runs its
// matrix phase while the other runs its softmax phase (vector ALU only), and
// the groups swap at the next barrier, so each SIMD has one wave feeding the
// matrix pipe while the other computes exponentials.
//
// A wave's step m is a matrix phase, S(m + 1) = K(m + 1) Q^T and
// O += P(m - 1) V(m - 1) (32 MFMAs at d = 128), then a softmax phase that
// turns S(m) into P(m).  S is computed one tile ahead (two S buffers): a
// wave's softmax reads S issued a full step earlier, which has left the
// matrix pipe whatever the other wave queued behind it.
//
// Staging: group A loads the K tiles, group B the V tiles, HBM -> LDS
// directly (no registers), into rings of four K and four V slots (160 KiB
// at d = 128); the loads of a matrix phase are spread over its k-steps.  A
// tile is published one half-step before the matrix phase that first reads
// it, so each wave reads that phase's first K and V^T fragments at the end
// of its softmax phase, and they land while it waits at the barrier: the
// phase opens with an MFMA instead of an LDS round trip.
//
// Launch: one workgroup per query tile, or persistent (persistent_task):
// one workgroup per CU that runs its share of the tiles one after another,
// which saves the gap between one workgroup's end and the next one's start
// on the CU (2-4 % on the 8k causal and the windowed workloads).
// ---------------------------------------------------------------------------

// Direct HBM -> LDS load of 16 bytes per lane (buffer_load ... lds): lane l
// writes LDS bytes lds_addr + 16 l .. + 15, lds_addr taken from M0.  Written
// as inline asm so that the compiler does not make every barrier and LDS
// read wait for these loads (it would treat each as an LDS store of unknown
// extent); the kernel waits for them itself with s_waitcnt vmcnt before the
// barrier that publishes the tile.  No register receives data.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds_addr,
                                          uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory");
}

// Workgroup barrier that leaves this wave's LDS reads in flight: the next
// matrix phase's first K and V^T fragments are read just before it and land
// while the wave waits.  s_barrier alone (no release fence, which would wait
// for them first); the memory clobber keeps the compiler from moving loads
// across it.  No wave writes the LDS with ordinary stores in this kernel, so
// the fence has nothing else to order.
__device__ __forceinline__ void barrier_keep_reads() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Wait until at most N of this wave's vector memory loads are outstanding.
template <int N>
__device__ __forceinline__ void wait_loads() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// A K or V tile in LDS, filled by direct loads: its padded rows (K: kCh + 1
// chunks of 16 bytes, V: kCh + 4) are laid end to end in a region of
// 64 (kCh + 4) chunks, which the 4 waves of a group fill with kWaveLoads
// wave-wide loads each (64 consecutive chunks per load).  Chunks that are
// row padding, or past the 64th row, load from outside the buffer (zero, no
// memory access).
template <int D>
struct DmaTile {
  using g = Geo<D>;
  static constexpr int kChunks = kBN * (g::kCh + 4);  // chunks per region
  static constexpr int kRegionB = kChunks * 16;
  static constexpr int kWaveLoads = kChunks / 256;    // per wave of a group of 4
  static_assert(kWaveLoads * 256 == kChunks, "region must split over 4 waves");
  static constexpr uint32_t kNowhere = 0x40000000u;   // beyond any slice

  uint32_t voff[kWaveLoads];

  // Global byte offsets (relative to the tile's first row) of this lane's
  // chunks; cpr = chunks per padded row.
  __device__ __forceinline__ void init(int cpr, int w4, int lane) {
#pragma unroll
    for (int i = 0; i < kWaveLoads; ++i) {
      const int s = 64 * (w4 + 4 * i) + lane;
      const int row = s / cpr, c = s - row * cpr;
      voff[i] = (c < g::kCh && row < kBN) ? (uint32_t)(row * g::kRowB + c * 16) : kNowhere;
    }
  }
  // Load i (0 .. kWaveLoads - 1) of this wave's share of the tile starting
  // at key row j0, into the region at LDS byte address region.
  __device__ __forceinline__ void issue_one(__amdgpu_buffer_rsrc_t rs, uint32_t region, int j0,
                                            int w4, int i) const {
    lds_dma16(rs, region + 1024u * (uint32_t)(w4 + 4 * i), voff[i], (uint32_t)j0 * g::kRowB);
  }
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, uint32_t region, int j0,
                                        int w4) const {
#pragma unroll
    for (int i = 0; i < kWaveLoads; ++i) issue_one(rs, region, j0, w4, i);
  }
};

// Online softmax of one tile, in place, scheduled for a wave that runs it
// alone on its SIMD's vector ALU (the other wave is issuing MFMAs): every
// step is a batch of independent instructions, so each result is used
// several instructions after it is produced.  The row max first (a max3
// tree; lazy reference move and rescale as in softmax_core, the rescale of
// O inside the rare branch), then p = exp2(c * s - m2) overwrites s, packed
// to bf16 as the B operand of the PV MFMAs, and the fp32 running sum (the
// sum of the bf16 weights is taken in the next matrix phase).
template <int KDB>
__device__ __forceinline__ void softmax_pp(f32x16 (&s)[2], bf16x8 (&pf)[2][2], RowState &st,
                                           f32x16 (&oacc)[KDB], float c) {
  auto S = [&](int i) { return s[i >> 4][i & 15]; };
  float a[10];
#pragma unroll
  for (int i = 0; i < 10; ++i) a[i] = fmaxf(fmaxf(S(3 * i), S(3 * i + 1)), S(3 * i + 2));
  float b3[4];
#pragma unroll
  for (int j = 0; j < 3; ++j) b3[j] = fmaxf(fmaxf(a[3 * j], a[3 * j + 1]), a[3 * j + 2]);
  b3[3] = fmaxf(fmaxf(a[9], S(30)), S(31));
  const float mx = fmaxf(fmaxf(fmaxf(b3[0], b3[1]), b3[2]), b3[3]);
  const float mt2 = wave_max_pair(mx) * c;
  if (__builtin_amdgcn_ballot_w64(mt2 > st.m2 + kTau) != 0) {
    const float mnew = fmaxf(st.m2, mt2);
    const float alpha = __builtin_amdgcn_exp2f(st.m2 - mnew);
    st.lsum *= alpha;
    st.lrnd *= alpha;
#pragma unroll
    for (int i = 0; i < KDB; ++i) oacc[i] *= alpha;
    st.m2 = mnew;
  }
  const float negm = -st.m2;
#pragma unroll
  for (int i = 0; i < 32; ++i) s[i >> 4][i & 15] = __builtin_fmaf(S(i), c, negm);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < 32; ++i) s[i >> 4][i & 15] = __builtin_amdgcn_exp2f(S(i));
  __builtin_amdgcn_sched_barrier(0);
  // register 8 tt + e of block rb is element e of pf[rb][tt]
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[rb][tt][e] = (__bf16)s[rb][8 * tt + e];
    }
  }
  float t[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) t[i] = S(2 * i) + S(2 * i + 1);
#pragma unroll
  for (int i = 0; i < 8; ++i) t[i] += t[i + 8];
#pragma unroll
  for (int i = 0; i < 4; ++i) t[i] += t[i + 4];
  t[0] += t[2];
  t[1] += t[3];
  st.lsum += t[0] + t[1];
}

// The matrix phase: S^T = K Q^T (DO_S) and O^T += V^T P^T (DO_PV),
// interleaved two MFMAs of each per k-step; hook(j) runs after the S MFMAs
// of k-step j (the tile loads, spread over the phase).  On entry ka[0], ka[1]
// hold the K fragments of k-steps 0 and 1 and va[0..3] the first four V^T
// fragments.
template <int D, bool DO_S, bool DO_PV, class Hook>
__device__ __forceinline__ void mfma_phase(const lchar *kb, const lchar *vb,
                                           const bf16x8 (&qf)[Geo<D>::kKSteps], f32x16 (&s)[2],
                                           const bf16x8 (&pf)[2][2],
                                           f32x16 (&oacc)[Geo<D>::kDB], bf16x8 (&ka)[3][2],
                                           bf16x8 (&va)[4], float &lrnd, Hook &&hook) {
  using g = Geo<D>;
  static_assert(g::kPV == 2 * g::kKSteps, "two PV MFMAs per S k-step");
  // The sum of the bf16 weights as the PV MFMAs use them (O is normalized by
  // it): one v_dot2 against (1, 1) per packed pair of weights, in four
  // partial sums.  The compiler issues them after the phase's last MFMA, in
  // its shadow; in the softmax phase they waited for the other wave's MFMAs,
  // and pinned between the MFMAs (one chain) the phase measured slower.
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float rp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  auto vf = [&](int i) { return vfrag<D>(vb, i >> 2, (i >> 1) & 1, i & 1); };
  if constexpr (DO_S) {
    s[0] = f32x16{};
    s[1] = f32x16{};
  }
#pragma unroll
  for (int j = 0; j < g::kKSteps; ++j) {
    hook(j);
    if constexpr (DO_S) {
      if (j + 2 < g::kKSteps) {
        ka[(j + 2) % 3][0] = kfrag<D>(kb, j + 2, 0);
        ka[(j + 2) % 3][1] = kfrag<D>(kb, j + 2, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[j % 3][0], qf[j], s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[j % 3][1], qf[j], s[1], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (DO_PV) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = 2 * j + u;
        const int db = i >> 2, rb = (i >> 1) & 1, tt = i & 1;
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i % 4], pf[rb][tt], oacc[db], 0, 0, 0);
        if (i + 4 < g::kPV) va[i % 4] = vf(i + 4);
#pragma unroll
        for (int t = 0; t < 16 / g::kPV; ++t) {  // pair n: word n % 4 of pf[n / 8][(n / 4) % 2]
          const int n = i * (16 / g::kPV) + t;
          const bf16x8 &w = pf[n >> 3][(n >> 2) & 1];
          const bf16x2 pair = {w[2 * (n & 3)], w[2 * (n & 3) + 1]};
          rp[n & 3] = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, rp[n & 3], false);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if constexpr (DO_PV) lrnd += (rp[0] + rp[1]) + (rp[2] + rp[3]);
}

// Persistent schedule (one workgroup per CU, each running several tiles in
// turn).  XCD x takes the head groups x, x + 8, ..., so every tile of a head
// reads its K/V behind one L2.  Its tiles are dealt to its S slots in
// rounds, alternately forwards and backwards, which evens out the causal
// work: in round r slot s takes tile k = r S + s (r even) or r S + S - 1 - s
// (r odd).  Tile k is, without a window, head k / nq, query tile rank
// k % nq (head by head, heaviest first within a head: the slots running at
// one time mostly share a head and stream the same K/V tiles from key 0
// up); with a window, rank k / hx of head k % hx (the ranks running at one
// time span fewer rows of each head, and so fewer keys).  Measured on
// MI355X: each order is 2-4 % faster than the other where it is used.
// Returns false when slot s has no tile in round r.
__device__ __forceinline__ bool persistent_task(const Params &prm, int r, int &qrank, int &hgb) {
  const int x = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int H = prm.B * prm.groups;
  const int hx = (H - x + 7) >> 3;  // head groups of XCD x
  const int S = prm.slots;
  const int k = r * S + ((r & 1) ? S - 1 - slot : slot);
  if (k >= prm.nq * hx) return false;
  int hl;
  if (prm.window > 0) {
    qrank = k / hx;
    hl = k - qrank * hx;
  } else {
    hl = k / prm.nq;
    qrank = k - hl * prm.nq;
  }
  hgb = hl * 8 + x;
  return true;
}

template <int D, int P, bool GEN>
__global__ __launch_bounds__(512, 2) void attn_fwd_pp_kernel(Params prm) {
  using g = Geo<D>;
  constexpr int kRows = 32 * 8 / P;  // query rows per workgroup
  using dt = DmaTile<D>;
  constexpr int kKSlots = 4;  // K ring
  constexpr int kVSlots = 4;  // V ring (8 slots: 160 KiB of LDS at d = 128)
  static_assert(g::kVTileB == dt::kRegionB, "a V tile fills its region");

  __shared__ __attribute__((aligned(1024))) char smem[(kKSlots + kVSlots) * dt::kRegionB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0: group A (stages K), 1: group B (stages V)
  const int l32 = lane & 31, hh = lane >> 5;

  // One query tile per pass: the workgroup's own in the one-workgroup-per-
  // tile launch (a single pass, straight-line code in the general mode), or
  // the persistent schedule's next.
  for (int r = 0; GEN ? r < 1 : true; ++r) {
    int pq = -1, ph = -1;
    if (GEN || prm.slots == 0) {
      if (r > 0) break;
    } else if (!persistent_task(prm, r, pq, ph)) {
      break;
    }
    const Task tk = make_task<P, kRows, GEN>(prm, wave, pq, ph);
    if (tk.empty) continue;  // the whole workgroup
    const int N = tk.N;
    const __amdgpu_buffer_rsrc_t rs_k = make_rsrc(prm.k + tk.kv_slice * D, (uint32_t)N * D * 2);
    const __amdgpu_buffer_rsrc_t rs_v = make_rsrc(prm.v + tk.kv_slice * D, (uint32_t)N * D * 2);

    bf16x8 qf[g::kKSteps];
    load_q<D>(prm, tk, l32, hh, qf);
    const int k_lane = k_lane_off<D>(lane);
    const int v_lane = v_lane_off<D>(lane);

    f32x16 oacc[g::kDB];
  #pragma unroll
    for (int i = 0; i < g::kDB; ++i) oacc[i] = f32x16{};
    RowState st;
    const float c = prm.c;
  #pragma unroll
    for (int kk = 0; kk < g::kKSteps; ++kk) asm volatile("" : "+v"(qf[kk]) : : "memory");

    const int count = tk.wg.count();
    auto row_of = [&](int k) { return k < count ? tk.wg.tile(k) * kBN : N; };
    auto ktile = [&](int j) { return (lchar *)smem + (j & (kKSlots - 1)) * dt::kRegionB; };
    auto vtile = [&](int j) {
      return (lchar *)smem + (kKSlots + (j & (kVSlots - 1))) * dt::kRegionB;
    };
    auto sees = [&](int m) { return m < count && tk.w.has(tk.wg.tile(m)); };

    // S of two tiles in flight: S(m) in sb[m % 2] is turned into weights while
    // the MFMAs of S(m + 1) run.
    f32x16 sb[2][2];
    bf16x8 pf[2][2];
    bf16x8 ka[3][2];
    bf16x8 va[4];

    // Group A stages K, group B stages V.
    auto group_program = [&](auto grp_c) {
      constexpr int G = decltype(grp_c)::value;
      const int w4 = wave & 3;
      // Half-step h: group A runs matrix(m) at h = 2m and vector(m) at
      // 2m + 1, group B one half-step later.  matrix(m) reads K(m + 1) and
      // V(m - 1); its first fragments are read at the end of the softmax
      // phase before it, so tile j must be published (loads landed, then a
      // barrier) one half-step before that: K(j) by the end of half-step
      // 2j - 4, V(j) by the end of 2j.  A slot's next tile is loaded
      // (straight into LDS) once both groups have read the previous one.
      // Group A loads K(m + 4) in its matrix phase of step m >= 1 (K(4) too in
      // step 1; K(0..3) before step 0) and waits for K(m + 2) at the end of
      // that phase; group B loads V(m + 2) in its matrix phase of step m and
      // waits for V(m + 1) at the end of its softmax phase of step m.  The
      // loads are spread over the phase's k-steps.  Loads past the last tile
      // read outside the buffer (zero, no memory access), so the number of
      // loads in flight does not depend on the tile count.
      const __amdgpu_buffer_rsrc_t rs = G == 0 ? rs_k : rs_v;
      dt dma;
      dma.init(G == 0 ? g::kCh + 1 : g::kCh + 4, w4, lane);
      auto region = [&](int j) { return (uint32_t)(uintptr_t)(G == 0 ? ktile(j) : vtile(j)); };
      if constexpr (G == 0) {
        dma.issue(rs, region(0), row_of(0), w4);
        dma.issue(rs, region(1), row_of(1), w4);
        dma.issue(rs, region(2), row_of(2), w4);
        dma.issue(rs, region(3), row_of(3), w4);
        wait_loads<2 * dt::kWaveLoads>();  // K(0), K(1)
        __syncthreads();
      } else {
        dma.issue(rs, region(0), row_of(0), w4);
        dma.issue(rs, region(1), row_of(1), w4);
        __syncthreads();
        wait_loads<dt::kWaveLoads>();  // V(0)
        __syncthreads();               // group B runs one half-step behind
      }

      // the loads of the matrix phase of step m, load i at k-step i
      auto loads = [&](int m) {
        return [&, m](int i) {
          if (i < dt::kWaveLoads) {
            if constexpr (G == 0) {
              if (m == 1) dma.issue_one(rs, region(4), row_of(4), w4, i);
              if (m >= 1) dma.issue_one(rs, region(m + 4), row_of(m + 4), w4, i);
            } else {
              dma.issue_one(rs, region(m + 2), row_of(m + 2), w4, i);
            }
          }
        };
      };
      auto no_loads = [](int) {};
      auto prefetch_k = [&](int j) {  // K fragments of k-steps 0, 1 of tile j
        const lchar *kb = ktile(j) + k_lane;
        ka[0][0] = kfrag<D>(kb, 0, 0);
        ka[0][1] = kfrag<D>(kb, 0, 1);
        ka[1][0] = kfrag<D>(kb, 1, 0);
        ka[1][1] = kfrag<D>(kb, 1, 1);
      };
      auto prefetch_v = [&](int j) {  // the first four V^T fragments of tile j
        const lchar *vb = vtile(j) + v_lane;
  #pragma unroll
        for (int i = 0; i < 4; ++i) va[i] = vfrag<D>(vb, i >> 2, (i >> 1) & 1, i & 1);
      };
      // Softmax phase of step m: weights P(m) from S(m) (zero if no row of
      // the wave sees tile m).
      auto vector = [&](int m, f32x16 (&s)[2]) {
        if (sees(m)) {
          mask_tile<GEN, true>(s, prm, tk.wg.tile(m) * kBN, tk.qw0, l32, hh, N);
          softmax_pp<g::kDB>(s, pf, st, oacc, c);
        } else {
  #pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
  #pragma unroll
            for (int tt = 0; tt < 2; ++tt) pf[rb][tt] = bf16x8{};
          }
        }
      };
      // End of the softmax phase of step m - 1: group B's loads of V(m) have
      // landed, and the first fragments of the matrix phase of step m are
      // read, left in flight across the barrier that ends the half-step.
      auto end_vector = [&](int m) {
        if constexpr (G == 1) wait_loads<dt::kWaveLoads>();  // V(m)
        __builtin_amdgcn_sched_barrier(0);
        prefetch_k(m + 1);
        prefetch_v(m - 1);
        barrier_keep_reads();
      };
      // Matrix phase of step m: S(m + 1) and O += P(m - 1) V(m - 1).  Every
      // wave runs the same MFMAs whatever its rows see (S of a tile past the
      // last is computed from whatever the slot holds and never used): one
      // code path keeps O in the same registers throughout.  The fragments
      // are read in the same block as the MFMAs that use them, so they are
      // not carried around the loop.
      auto matrix = [&](int m, f32x16 (&s_next)[2]) {
        end_vector(m);
        __builtin_amdgcn_s_setprio(2);
        mfma_phase<D, true, true>(ktile(m + 1) + k_lane, vtile(m - 1) + v_lane, qf, s_next, pf,
                                  oacc, ka, va, st.lrnd, loads(m));
        __builtin_amdgcn_s_setprio(0);
        if constexpr (G == 0) wait_loads<2 * dt::kWaveLoads>();  // K(m + 2)
        __syncthreads();
      };

      // step 0: S(0) and S(1)
      __builtin_amdgcn_s_setprio(2);
      prefetch_k(0);
      mfma_phase<D, true, false>(ktile(0) + k_lane, nullptr, qf, sb[0], pf, oacc, ka, va,
                                 st.lrnd, loads(0));
      prefetch_k(1);
      mfma_phase<D, true, false>(ktile(1) + k_lane, nullptr, qf, sb[1], pf, oacc, ka, va,
                                 st.lrnd, no_loads);
      __builtin_amdgcn_s_setprio(0);
      if constexpr (G == 0) wait_loads<dt::kWaveLoads>();  // K(2)
      __syncthreads();
      vector(0, sb[0]);
      int m = 1;
      for (;;) {
        if (m == count) break;
        matrix(m, sb[0]);  // S(m + 1), m odd
        vector(m, sb[1]);
        ++m;
        if (m == count) break;
        matrix(m, sb[1]);  // S(m + 1), m even
        vector(m, sb[0]);
        ++m;
      }
      // last step: O += P(count - 1) V(count - 1), its first V^T fragments
      // read at the end of the last softmax phase (the K fragments read there
      // are not used)
      end_vector(count);
      __builtin_amdgcn_s_setprio(2);
      mfma_phase<D, false, true>(nullptr, vtile(count - 1) + v_lane, qf, sb[0], pf, oacc, ka, va,
                                 st.lrnd, no_loads);
      __builtin_amdgcn_s_setprio(0);
      __syncthreads();
      if (G == 0) __syncthreads();
    };
    if (grp == 0) {
      group_program(std::integral_constant<int, 0>{});
    } else {
      group_program(std::integral_constant<int, 1>{});
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load left in flight

    write_out<D>(prm, tk, l32, hh, oacc, st);
    // every wave has passed the tile's last barrier, after its last LDS read:
    // the next tile's loads may overwrite the rings
  }
}

// Compute units of the current device (cached per device).
int device_cus() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cus[dev] = n;
  }
  return cus[dev];
}

template <int D, int P>
hipError_t launch_pp_t(const FwdProblem &p, hipStream_t stream, bool persistent) {
  constexpr int kRows = 32 * 8 / P;
  Params prm{};
  prm.q = static_cast<const uint16_t *>(p.q);
  prm.k = static_cast<const uint16_t *>(p.k);
  prm.v = static_cast<const uint16_t *>(p.v);
  prm.o = static_cast<uint16_t *>(p.o);
  prm.lse = p.lse;
  prm.B = p.B; prm.Hq = p.Hq; prm.Hkv = p.Hkv; prm.N = p.N;
  prm.G = p.Hq / p.Hkv;
  prm.groups = p.Hq / P;
  prm.nq = (p.N + kRows - 1) / kRows;
  const long long total = (long long)p.B * prm.groups * prm.nq;
  if (total > 0x7fffffffLL) return hipErrorInvalidValue;
  prm.total = (int)total;
  prm.nkt = (p.N + kBN - 1) / kBN;
  const float c = std::fabs(p.scale) * kLog2e;
  prm.c = c < FLT_MIN ? FLT_MIN : c;
  prm.neg = p.scale < 0.0f ? 1 : 0;
  prm.causal = p.causal;
  prm.window = p.window;
  // persistent: one workgroup per CU, when every XCD has a head group and
  // every slot at least two tiles
  const int slots = device_cus() / 8;
  unsigned grid = prm.total;
  if (persistent && slots > 0 && p.B * prm.groups >= 8 && prm.total >= 16 * slots) {
    prm.slots = slots;
    grid = 8 * slots;
  }
  void *args[] = {&prm};
  return hipLaunchKernel(reinterpret_cast<const void *>(&attn_fwd_pp_kernel<D, P, false>),
                         dim3(grid), dim3(512), args, 0, stream);
}

template <int D>
hipError_t launch_pp(const FwdProblem &p, hipStream_t stream, bool persistent) {
  const int G = p.Hq / p.Hkv;
  if (G % 8 == 0) return launch_pp_t<D, 8>(p, stream, persistent);
  if (G % 4 == 0) return launch_pp_t<D, 4>(p, stream, persistent);
  if (G % 2 == 0) return launch_pp_t<D, 2>(p, stream, persistent);
  return launch_pp_t<D, 1>(p, stream, persistent);
}

template <int D, int NW, int P>
hipError_t launch_t(const FwdProblem &p, hipStream_t stream) {
  constexpr int kRows = 32 * NW / P;
  Params prm{};
  prm.q = static_cast<const uint16_t *>(p.q);
  prm.k = static_cast<const uint16_t *>(p.k);
  prm.v = static_cast<const uint16_t *>(p.v);
  prm.o = static_cast<uint16_t *>(p.o);
  prm.lse = p.lse;
  prm.B = p.B; prm.Hq = p.Hq; prm.Hkv = p.Hkv; prm.N = p.N;
  prm.G = p.Hq / p.Hkv;
  prm.groups = p.Hq / P;
  prm.nq = (p.N + kRows - 1) / kRows;
  const long long total = (long long)p.B * prm.groups * prm.nq;
  if (total > 0x7fffffffLL) return hipErrorInvalidValue;
  prm.total = (int)total;
  prm.nkt = (p.N + kBN - 1) / kBN;
  const float c = std::fabs(p.scale) * kLog2e;
  prm.c = c < FLT_MIN ? FLT_MIN : c;
  prm.neg = p.scale < 0.0f ? 1 : 0;
  prm.causal = p.causal;
  prm.window = p.window;
  void *args[] = {&prm};
  return hipLaunchKernel(reinterpret_cast<const void *>(&attn_fwd_kernel<D, NW, P, false>),
                         dim3(prm.total), dim3(NW * 64), args, 0, stream);
}

// Waves per workgroup of the general (packed, structured-mask) kernels:
// at d = 64 three 4-wave workgroups share a CU (138 VGPRs, 43 KB of LDS),
// and their waves, not held together by one barrier, overlap one another's
// softmax and matrix products; at d = 128 one 8-wave workgroup per CU.
template <int D>
constexpr int kGenWaves = D == 64 ? 4 : 8;

template <int D, int P>
hipError_t launch_gen_t(const VarlenProblem &p, hipStream_t stream) {
  constexpr int NW = kGenWaves<D>;
  constexpr int kRows = 32 * NW / P;
  Params prm{};
  prm.q = static_cast<const uint16_t *>(p.q);
  prm.k = static_cast<const uint16_t *>(p.k);
  prm.v = static_cast<const uint16_t *>(p.v);
  prm.o = static_cast<uint16_t *>(p.o);
  prm.lse = p.lse;
  prm.B = p.B; prm.Hq = p.Hq; prm.Hkv = p.Hkv; prm.N = p.max_seqlen;
  prm.G = p.Hq / p.Hkv;
  prm.groups = p.Hq / P;
  prm.nq = (p.max_seqlen + kRows - 1) / kRows;
  const long long total = (long long)p.B * prm.groups * prm.nq;
  if (total > 0x7fffffffLL) return hipErrorInvalidValue;
  prm.total = (int)total;
  prm.nkt = (p.max_seqlen + kBN - 1) / kBN;
  const float c = std::fabs(p.scale) * kLog2e;
  prm.c = c < FLT_MIN ? FLT_MIN : c;
  prm.neg = p.scale < 0.0f ? 1 : 0;
  prm.causal = p.causal;
  prm.window = p.window;
  prm.cu = p.cu_seqlens;
  prm.total_rows = p.total_rows;
  prm.radius = p.radius;
  prm.nglob = p.n_global;
  prm.compact = (long long)p.B * p.max_seqlen != p.total_rows;
  // global rows: workgroups of their own, placed first in the launch
  if (p.n_global > 0) {
    const long long ngt = (long long)p.B * p.Hq * ((p.n_global + 31) / 32);
    if (ngt + prm.total > 0x7fffffffLL) return hipErrorInvalidValue;
    prm.gsplit = 1;
    prm.ngtask = (int)ngt;
  }
  void *args[] = {&prm};
  return hipLaunchKernel(reinterpret_cast<const void *>(&attn_fwd_kernel<D, NW, P, true>),
                         dim3(prm.total + prm.ngtask), dim3(NW * 64), args, 0, stream);
}

template <int D, int P>
hipError_t launch_gen_pp_t(const VarlenProblem &p, hipStream_t stream) {
  constexpr int kRows = 32 * 8 / P;
  Params prm{};
  prm.q = static_cast<const uint16_t *>(p.q);
  prm.k = static_cast<const uint16_t *>(p.k);
  prm.v = static_cast<const uint16_t *>(p.v);
  prm.o = static_cast<uint16_t *>(p.o);
  prm.lse = p.lse;
  prm.B = p.B; prm.Hq = p.Hq; prm.Hkv = p.Hkv; prm.N = p.max_seqlen;
  prm.G = p.Hq / p.Hkv;
  prm.groups = p.Hq / P;
  prm.nq = (p.max_seqlen + kRows - 1) / kRows;
  const long long total = (long long)p.B * prm.groups * prm.nq;
  if (total > 0x7fffffffLL) return hipErrorInvalidValue;
  prm.total = (int)total;
  prm.nkt = (p.max_seqlen + kBN - 1) / kBN;
  const float c = std::fabs(p.scale) * kLog2e;
  prm.c = c < FLT_MIN ? FLT_MIN : c;
  prm.neg = p.scale < 0.0f ? 1 : 0;
  prm.causal = p.causal;
  prm.window = p.window;
  prm.cu = p.cu_seqlens;
  prm.total_rows = p.total_rows;
  prm.radius = p.radius;
  prm.nglob = p.n_global;
  prm.compact = (long long)p.B * p.max_seqlen != p.total_rows;
  void *args[] = {&prm};
  return hipLaunchKernel(reinterpret_cast<const void *>(&attn_fwd_pp_kernel<D, P, true>),
                         dim3(prm.total), dim3(512), args, 0, stream);
}

template <int D>
hipError_t launch_gen_d(const VarlenProblem &p, hipStream_t stream) {
  const int G = p.Hq / p.Hkv;
  if constexpr (D == 128) {  // the ping-pong kernel, as the dense default, without global rows
    if (p.n_global == 0) {
      if (G % 8 == 0) return launch_gen_pp_t<D, 8>(p, stream);
      if (G % 4 == 0) return launch_gen_pp_t<D, 4>(p, stream);
      if (G % 2 == 0) return launch_gen_pp_t<D, 2>(p, stream);
      return launch_gen_pp_t<D, 1>(p, stream);
    }
  }
  if constexpr (kGenWaves<D> >= 8) {
    if (G % 8 == 0) return launch_gen_t<D, 8>(p, stream);
  }
  if (G % 4 == 0) return launch_gen_t<D, 4>(p, stream);
  if (G % 2 == 0) return launch_gen_t<D, 2>(p, stream);
  return launch_gen_t<D, 1>(p, stream);
}

template <int D, int NW>
hipError_t launch_nw(const FwdProblem &p, hipStream_t stream) {
  const int G = p.Hq / p.Hkv;
  // heads packed per workgroup: the largest power of two <= NW dividing G
  if constexpr (NW >= 8) {
    if (G % 8 == 0) return launch_t<D, NW, 8>(p, stream);
  }
  if (G % 4 == 0) return launch_t<D, NW, 4>(p, stream);
  if (G % 2 == 0) return launch_t<D, NW, 2>(p, stream);
  return launch_t<D, NW, 1>(p, stream);
}

template <int D>
hipError_t launch_d(const FwdProblem &p, int v, hipStream_t stream) {
  if (v == kPingPong || v == kPersistent) return launch_pp<D>(p, stream, v == kPersistent);
  return v == kWaves4 ? launch_nw<D, 4>(p, stream) : launch_nw<D, 8>(p, stream);
}

}  // namespace

const char *variant_name(int variant) {
  switch (variant) {
    case kAuto: return "auto";
    case kWaves4: return "w4_bn64_mfma32x32x16";
    case kWaves8: return "w8_bn64_mfma32x32x16";
    case kPingPong: return "w8_pingpong_bn64_mfma32x32x16";
    case kPersistent: return "w8_pingpong_persistent_bn64_mfma32x32x16";
  }
  return "invalid";
}

hipError_t launch_fwd(const FwdProblem &p, int variant, hipStream_t stream) {
  // default: at d = 128 the ping-pong kernel, persistent (one workgroup per
  // CU) when the problem has enough tiles; at d = 64 the 4-wave lockstep
  // kernel, where 138 VGPRs let three 4-wave workgroups share a CU
  const int v = variant != kAuto ? variant : p.d == 64 ? kWaves4 : kPersistent;
  return p.d == 128 ? launch_d<128>(p, v, stream) : launch_d<64>(p, v, stream);
}

hipError_t launch_fwd_varlen(const VarlenProblem &p, hipStream_t stream) {
  return p.d == 128 ? launch_gen_d<128>(p, stream) : launch_gen_d<64>(p, stream);
}

}  // namespace attn
