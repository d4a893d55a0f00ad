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
// no row of a wave can see are never visited ("Against the real libraries":
// mask structure becomes loop bounds).
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
// * K and V tiles go HBM -> registers -> LDS, 16 bytes per lane per load,
//   double-buffered: the loads of tile t+1 are issued before tile t is
//   computed and written to the other LDS buffer after it, so their latency
//   hides behind a whole tile of MFMAs.  (Direct buffer_load ... lds would
//   save the registers, but the compiler then waits for every outstanding
//   vector load before each transposed LDS read.)  The buffer descriptor
//   spans one (batch, KV-head) slice, so keys past N read as zero.  Inside a
//   row the 16-byte chunks are XOR-swizzled so that both the b128 K reads
//   and the transposed V reads hit distinct LDS banks.
// * GQA: the query heads sharing a KV head are packed into one workgroup
//   (one head per wave), so each K/V tile is loaded once for all of them.
// * The running max is exact.  When no row of the wave gets a larger max
//   from a tile (the common case once a row has seen a few tiles), the
//   rescale of the O accumulator is skipped with one wave-uniform branch.
//   An exact max keeps the largest weight of every row at exactly 1.0, so
//   the bf16 rounding of P never touches the dominant term of a sharp row.

#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstdint>

#include "attn_internal.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((vector_size(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8_t;

constexpr int kBN = 64;              // keys per tile
constexpr float kTau = 8.0f;         // lazy-rescale threshold, log2 units
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kBufferFlags = 0x00020000;  // gfx9 buffer descriptor word 3

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
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kBufferFlags);
}

// Workgroup id -> logical id.  Consecutive hardware ids are dealt round-robin
// to the 8 XCDs; this gives XCD x one contiguous range of logical ids, so the
// workgroups sharing one head's K/V run behind one L2.
__device__ __forceinline__ int xcd_remap(int id, int total) {
  const int q = total >> 3, r = total & 7;
  const int x = id & 7, slot = id >> 3;
  return x < r ? x * (q + 1) + slot : r * (q + 1) + (x - r) * q + slot;
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef char __attribute__((address_space(3))) lchar;

// This thread's share of one K or V tile: kLoads 16-byte chunks.  Chunk
// n covers tile row r = ci / kCh, chunk p = ci % kCh with
// ci = n * NW * 64 + tid, so each wave instruction reads whole rows
// contiguously from HBM.  Keys past N read as zero (buffer range check).
template <int D, int NW>
struct TileStage {
  using g = Geo<D>;
  static constexpr int kLoads = kBN * g::kCh / (NW * 64);
  static_assert(kLoads * NW * 64 == kBN * g::kCh, "tile must split evenly over the threads");
  u32x4 k[kLoads], v[kLoads];

  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, int j0,
                                       int tid) {
#pragma unroll
    for (int n = 0; n < kLoads; ++n) {
      const int ci = n * NW * 64 + tid;
      const int voff = j0 * g::kRowB + ci * 16;
      k[n] = __builtin_amdgcn_raw_buffer_load_b128(rk, voff, 0, 0);
      v[n] = __builtin_amdgcn_raw_buffer_load_b128(rv, voff, 0, 0);
    }
  }
  // Write into an LDS buffer set: the K tile at offset 0, the V tile at
  // kKTileB, each row at its padded stride.
  __device__ __forceinline__ void store(lchar *set, int tid) const {
    const int r0 = tid / g::kCh, p = tid % g::kCh;
    lchar *kp = set + r0 * g::kKStride + p * 16;
    lchar *vp = set + g::kKTileB + r0 * g::kVStride + p * 16;
    constexpr int kRowsPerLoad = NW * 64 / g::kCh;
#pragma unroll
    for (int n = 0; n < kLoads; ++n) {
      *(__attribute__((address_space(3))) u32x4 *)(kp + n * kRowsPerLoad * g::kKStride) = k[n];
      *(__attribute__((address_space(3))) u32x4 *)(vp + n * kRowsPerLoad * g::kVStride) = v[n];
    }
  }
};

__device__ __forceinline__ float wave_max_pair(float x) {
  // max of this lane and lane ^ 32
  auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float wave_sum_pair(float x) {
  auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

template <int D, int NW, int P>
__global__ __launch_bounds__(NW * 64, 2) void attn_fwd_kernel(Params prm) {
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

  // ---- which (batch, head, rows) this workgroup and wave own
  const int logical = xcd_remap(blockIdx.x, prm.total);
  const int qrank = logical % prm.nq;
  const int hgb = logical / prm.nq;
  const int hg = hgb % prm.groups, b = hgb / prm.groups;
  const int qi = prm.causal ? (prm.nq - 1 - qrank) : qrank;  // heaviest tiles first
  const int head = hg * P + (wave % P);
  const int kvh = __builtin_amdgcn_readfirstlane((hg * P) / prm.G);
  const int wg_r0 = qi * kRows;
  const int qw0 = wg_r0 + (wave / P) * 32;  // first row of this wave
  const int N = prm.N;

  // key-tile ranges: workgroup (union over its rows) and this wave
  auto tile_range = [&](int r0, int r1, int &lo, int &hi) {  // rows [r0, r1)
    hi = prm.causal ? min(prm.nkt, (r1 - 1) / kBN + 1) : prm.nkt;
    lo = prm.window > 0 ? max(0, r0 - prm.window + 1) / kBN : 0;
  };
  int wg_lo, wg_hi, w_lo, w_hi;
  tile_range(wg_r0, min(N, wg_r0 + kRows), wg_lo, wg_hi);
  if (qw0 < N) {
    tile_range(qw0, min(N, qw0 + 32), w_lo, w_hi);
  } else {
    w_lo = w_hi = 0;  // rows past the end: this wave only helps load tiles
  }

  // every wave of the workgroup reads the same KV head (P divides G)
  const size_t kv_slice = (size_t)(b * prm.Hkv + kvh) * N * D;
  const size_t q_slice = (size_t)(b * prm.Hq + head) * N * D;
  const __amdgpu_buffer_rsrc_t rs_k = make_rsrc(prm.k + kv_slice, (uint32_t)N * D * 2);
  const __amdgpu_buffer_rsrc_t rs_v = make_rsrc(prm.v + kv_slice, (uint32_t)N * D * 2);

  // ---- Q^T operand: lane holds query row qw0 + l32, d = 16*kk + 8*hh + s
  bf16x8 qf[g::kKSteps];
  {
    const int row = qw0 + l32;
    const uint16_t *qp = prm.q + q_slice + (size_t)row * D + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < g::kKSteps; ++kk) {
      if (row < N) {
        qf[kk] = *(const bf16x8 *)(qp + 16 * kk);
      } else {
        qf[kk] = bf16x8{};
      }
      if (prm.neg) {
        typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
        u32x4 t = __builtin_bit_cast(u32x4, qf[kk]);
        t ^= 0x80008000u;
        qf[kk] = __builtin_bit_cast(bf16x8, t);
      }
    }
  }

  // per-lane LDS byte offsets
  // K (b128): key row 32*rb + l32, d = 16*kk + 8*hh .. +7
  const int k_lane = l32 * g::kKStride + hh * 16;
  // V (transposed read): key row 32rb + 16tt + 8u + 4hh + (lane & 15) / 4,
  // d = 32db + 16*((lane >> 4) & 1) + 4*(lane & 3) .. +3
  const int v_lane = (4 * hh + ((lane & 15) >> 2)) * g::kVStride +
                     (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;

  f32x16 oacc[g::kDB];
#pragma unroll
  for (int i = 0; i < g::kDB; ++i) oacc[i] = f32x16{};
  float m2 = -1e30f;   // running max, scaled log2 units (finite: no inf - inf)
  float lsum = 0.0f;   // this lane's partial row sum (its 32 of every 64 keys)
  float lrnd = 0.0f;   // the same over the bf16-rounded weights
  const float c = prm.c;

  TileStage<D, NW> stage;
  if (wg_lo < wg_hi) {
    stage.load(rs_k, rs_v, wg_lo * kBN, tid);
    stage.store(set0, tid);
  }
  __syncthreads();

  // S^T, mask, online softmax and O^T update for key tile t held in `set`.
  auto compute = [&](const int t, const lchar *const set) {

    const int j0 = t * kBN;
    const lchar *kb = set + k_lane;
    const lchar *vb = set + g::kKTileB + v_lane;

    // LDS fragment readers.  K fragment (kk, rb): key row 32*rb + l32, d
    // chunk 2*kk + hh.  V^T fragment i of the PV sequence (db = i / 4,
    // rb = (i / 2) % 2, tt = i % 2): two transposed reads of 4 keys each.
    auto kfrag = [&](int kk, int rb) -> bf16x8 {
      return *(const lds_bf16x8_t *)(kb + rb * 32 * g::kKStride + kk * 32);
    };
    auto vfrag = [&](int i) -> bf16x8 {
      const int db = i >> 2, rb = (i >> 1) & 1, tt = i & 1;
      i16x4 half[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int off = (32 * rb + 16 * tt + 8 * u) * g::kVStride + db * 64;
        half[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(vb + off));
      }
      typedef short i16x8 __attribute__((ext_vector_type(8)));
      const i16x8 both = {half[0][0], half[0][1], half[0][2], half[0][3],
                          half[1][0], half[1][1], half[1][2], half[1][3]};
      return __builtin_bit_cast(bf16x8, both);
    };
    constexpr int kPV = 4 * g::kDB;  // PV MFMAs per tile
    constexpr int kKA = 3;           // K ring depth (k-steps in flight)
    constexpr int kVA = 4;           // V ring depth (MFMAs in flight)

    // ---- S^T = K Q^T for 64 keys x 32 queries; K reads run kKA-1 k-steps
    // ahead of the MFMAs that consume them (sched_barrier fences keep the
    // compiler from sinking each read onto its MFMA, which would expose the
    // full LDS latency on every MFMA).
    f32x16 s[2] = {f32x16{}, f32x16{}};
    bf16x8 ka[kKA][2];
#pragma unroll
    for (int kk = 0; kk < kKA - 1; ++kk) {
      ka[kk][0] = kfrag(kk, 0);
      ka[kk][1] = kfrag(kk, 1);
    }
#pragma unroll
    for (int kk = 0; kk < g::kKSteps; ++kk) {
      if (kk + kKA - 1 < g::kKSteps) {
        ka[(kk + kKA - 1) % kKA][0] = kfrag(kk + kKA - 1, 0);
        ka[(kk + kKA - 1) % kKA][1] = kfrag(kk + kKA - 1, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk % kKA][0], qf[kk], s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk % kKA][1], qf[kk], s[1], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the first V^T fragments do not depend on P: start them now so the
    // softmax hides their latency
    bf16x8 va[kVA];
#pragma unroll
    for (int i = 0; i < kVA; ++i) va[i] = vfrag(i);
    __builtin_amdgcn_sched_barrier(0);

    // ---- mask: only tiles that hold a masked (row, key) pair for this wave
    const bool need_mask = (prm.causal && j0 + kBN - 1 > qw0) ||
                           (prm.window > 0 && j0 <= qw0 + 31 - prm.window) || (j0 + kBN > N);
    if (need_mask) {
      // Register r of block rb holds key kbase + off with the compile-time
      // off = 32*rb + 8*(r/4) + r%4.  The keys this lane's row sees form the
      // range lo < off <= hi relative to kbase, so one unsigned compare per
      // register decides visibility: (unsigned)(off - lo - 1) < hi - lo.
      const int qrow = qw0 + l32;
      const int kbase = j0 + 4 * hh;
      int hi = N - 1 - kbase;
      if (prm.causal) hi = min(hi, qrow - kbase);
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
    }

    // ---- online softmax (scaled log2 domain)
    float mx = s[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    mx = wave_max_pair(mx);
    const float mt2 = mx * c;
    // Lazy rescale: the reference point m2 only moves (and O is rescaled)
    // when some row's tile max exceeds it by more than kTau (log2 units), so
    // P <= 2^kTau; most tiles skip the 64 multiplies.  When it moves, every
    // row of the wave takes its exact running max.
    const bool grow = mt2 > m2 + kTau;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float mnew = fmaxf(m2, mt2);
      const float alpha = __builtin_amdgcn_exp2f(m2 - mnew);
      lsum *= alpha;
      lrnd *= alpha;
#pragma unroll
      for (int i = 0; i < g::kDB; ++i) oacc[i] *= alpha;
      m2 = mnew;
    }
    const float negm = -m2;
    bf16x8 pf[2][2];
    float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // independent add chains
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
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
    lsum += (part[0] + part[1]) + (part[2] + part[3]);
    // The same weights as the PV MFMA sees them (bf16), summed with
    // v_dot2_f32_bf16 against (1, 1): normalizing O by this sum makes a row
    // dominated by one key return that key's V row up to fp32 rounding, even
    // when its weight is not exactly 1.0 (lazy rescale).
    {
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
      float rp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bf16x2 pair = {pf[rb][tt][2 * e], pf[rb][tt][2 * e + 1]};
            rp[e] = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, rp[e], false);
          }
        }
      }
      lrnd += (rp[0] + rp[1]) + (rp[2] + rp[3]);
    }

    // ---- O^T += V^T P^T; V reads run kVA MFMAs ahead
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kPV; ++i) {
      const int db = i >> 2, rb = (i >> 1) & 1, tt = i & 1;
      const bf16x8 a = va[i % kVA];
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[rb][tt], oacc[db], 0, 0, 0);
      if (i + kVA < kPV) va[i % kVA] = vfrag(i + kVA);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // One key tile: start loading the next tile into registers, compute this
  // one from LDS (if this wave sees any of its keys), then park the next tile
  // in the other buffer set.  The register loads are only waited for at that
  // final store, so they overlap the whole tile's compute.
  auto step = [&](const int t, lchar *const cur_set, lchar *const next_set) {
    const bool more = t + 1 < wg_hi;
    if (more) stage.load(rs_k, rs_v, (t + 1) * kBN, tid);
    if (t >= w_lo && t < w_hi) compute(t, cur_set);
    if (more) stage.store(next_set, tid);
    __syncthreads();
  };

  for (int t = wg_lo; t < wg_hi; t += 2) {
    step(t, set0, set1);
    if (t + 1 < wg_hi) step(t + 1, set1, set0);
  }

  // ---- epilogue: O = O / l (bf16, RNE), lse = ln(sum) + max
  const float ltot = wave_sum_pair(lsum);
  const float lrtot = wave_sum_pair(lrnd);
  const int row = qw0 + l32;
  if (row < N) {
    const float inv = 1.0f / lrtot;
    uint16_t *op = prm.o + q_slice + (size_t)row * D + 4 * hh;
#pragma unroll
    for (int db = 0; db < g::kDB; ++db) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = (__bf16)(oacc[db][4 * i + j] * inv);
        *(bf16x4 *)(op + 32 * db + 8 * i) = w;
      }
    }
    if (hh == 0) {
      prm.lse[(size_t)(b * prm.Hq + head) * N + row] = (m2 + __builtin_amdgcn_logf(ltot)) * kLn2;
    }
  }
}

template <int D, int NW, int P>
hipError_t launch_t(const FwdProblem &p, hipStream_t stream) {
  constexpr int kRows = 32 * NW / P;
  Params prm;
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
  return hipLaunchKernel(reinterpret_cast<const void *>(&attn_fwd_kernel<D, NW, P>),
                         dim3(prm.total), dim3(NW * 64), args, 0, stream);
}

template <int D, int NW>
hipError_t launch_nw(const FwdProblem &p, hipStream_t stream) {
  const int G = p.Hq / p.Hkv;
  // heads packed per workgroup: the largest power of two <= NW dividing G
  if (NW >= 8 && G % 8 == 0) return launch_t<D, NW, (NW >= 8 ? 8 : 1)>(p, stream);
  if (G % 4 == 0) return launch_t<D, NW, 4>(p, stream);
  if (G % 2 == 0) return launch_t<D, NW, 2>(p, stream);
  return launch_t<D, NW, 1>(p, stream);
}

}  // namespace

const char *variant_name(int variant) {
  switch (variant) {
    case kAuto: return "auto";
    case kWaves4: return "w4_bn64_mfma32x32x16";
    case kWaves8: return "w8_bn64_mfma32x32x16";
  }
  return "invalid";
}

hipError_t launch_fwd(const FwdProblem &p, int variant, hipStream_t stream) {
  const int v = variant == kAuto ? kWaves8 : variant;
  if (p.d == 128) {
    return v == kWaves4 ? launch_nw<128, 4>(p, stream) : launch_nw<128, 8>(p, stream);
  }
  return v == kWaves4 ? launch_nw<64, 4>(p, stream) : launch_nw<64, 8>(p, stream);
}

}  // namespace attn
