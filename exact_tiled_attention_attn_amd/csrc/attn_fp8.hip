// gfx950 (MI355X, CDNA4) FP8 attention forward and its input packing.
//
// What is computed: the exact attention of the dequantised FP8 tensors
// (the forward's definition; "Efficient attention: long context and
// sub-quadratic variants", section "FlashAttention: exact attention,
// IO-aware", attaches an FP8 path to FlashAttention-3).  Format OCP E4M3
// (bias 7, max 448, round to nearest even); one power-of-two scale per
// tensor, s = 2^e with e the smallest integer such that amax <= 448 * 2^e,
// so x / s is exact and never saturates.
//
// Packing (attn_fp8_quantize): an amax pass over Q, K, V (atomic max of the
// magnitudes' bit patterns), then Q and K become e4m3 codes in their own
// layout and V is written transposed, [B][Hkv][D][Np] (Np = N rounded up to
// 64), with the keys of each 64-key tile in the order the P^T operand holds
// them (key_of), so that V^T is read with plain b128 LDS reads.
//
// Forward (attn_fwd_fp8): the bf16 forward's lockstep tiling (workgroups of
// kF8Waves = 4 waves x 32 query rows, three workgroups per CU, 64-key tiles
// double-buffered through LDS, one query per lane), with
// v_mfma_scale_f32_32x32x64_f8f6f4: S^T = K Q^T takes
// D / 64 products per 32 keys and O^T += V^T P^T one product per 32 d
// values.  The weights are P' = 2^4 exp2(c s - m) against a lazily moved
// reference max m (it moves when a row's tile max exceeds it by more than 4
// log2 units, and only then is O rescaled), so P' <= 256 fits e4m3 and
// weights down to 2^-10 of the reference keep normal e4m3 precision; P' is
// rounded to e4m3 (RNE) for the product.
// The descales s_q s_k enter the exponent factor c, s_v the epilogue.

#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstdint>

#include "attn_device.h"
#include "attn_internal.h"

namespace attn {
namespace {

using namespace dev;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i32x4 lds_i32x4_t;

constexpr int kBN8 = 64;          // keys per tile
// Weights P' = 2^kPShift exp2(c s - m) against a reference max m that
// moves only when a row's tile max exceeds it by more than kTau8 (log2
// units), so P' <= 2^(kPShift + kTau8) = 256 <= 448 fits e4m3, and weights
// down to 2^-(6 + kPShift) of the reference keep normal e4m3 precision.
constexpr float kPShift = 4.0f;
// Waves per workgroup.  With 4 (166 VGPRs, 38 KB of LDS) three workgroups
// share a CU, and waves of different workgroups, not held together by a
// barrier, run their softmax while others run their matrix products: 3-8 %
// faster than one 8-wave workgroup per CU on the causal workloads.
constexpr int kF8Waves = 4;
constexpr float kTau8 = 4.0f;

// Key (0..63) of a 64-key tile held at byte b (0..31) of lane half h of the
// P^T operand: the S^T accumulators of key block rb = b / 16 hold, in
// register r = b % 16, key 32 rb + 8 (r / 4) + 4 h + r % 4.
__host__ __device__ constexpr int key_of(int h, int b) {
  return 32 * (b >> 4) + 8 * ((b & 15) >> 2) + 4 * h + (b & 3);
}

__device__ __forceinline__ f32x16 mfma8(const i32x8 &a, const i32x8 &b, const f32x16 &c) {
  // fp8 e4m3 x fp8 e4m3, no block scales (scale exponent 127 = 2^0)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Per-tensor power-of-two scale from its amax (exact, no division).
__device__ __forceinline__ int pow2_exp(float amax) {
  if (!(amax > 0.0f)) return 0;
  int E;
  const float f = frexpf(amax, &E);  // amax = f 2^E, 448 = 0.875 2^9
  return f <= 0.875f ? E - 9 : E - 8;
}

// ---------------------------------------------------------------------------
// packing
// ---------------------------------------------------------------------------
struct PackParams {
  const uint16_t *x[3];   // q, k, v (bf16)
  uint8_t *q8, *k8, *vt8;
  float *scales;          // [0..2] scales, [3..5] amax
  long long n[3];         // elements of q, k, v
  int B, Hkv, N, Np;
};

__global__ void attn_fp8_clear_kernel(float *scales) {
  if (threadIdx.x < 6) scales[threadIdx.x] = 0.0f;
}

// amax of tensor blockIdx.y: four independent 16-byte loads per thread per
// step keep enough reads in flight to run near the HBM rate
__global__ __launch_bounds__(256) void attn_fp8_amax_kernel(PackParams pp) {
  const int t = blockIdx.y;
  const bf16x8 *x = reinterpret_cast<const bf16x8 *>(pp.x[t]);
  const long long n8 = pp.n[t] / 8;
  const long long stride = (long long)gridDim.x * blockDim.x;
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  float m = 0.0f;
  for (; i + 3 * stride < n8; i += 4 * stride) {
    bf16x8 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(&x[i + u * stride]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf((float)v[u][e]));
  }
  for (; i < n8; i += stride) {
    const bf16x8 v = __builtin_nontemporal_load(&x[i]);
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf((float)v[e]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  // one atomic per workgroup: atomics on one address serialise, and every
  // workgroup reaches this point at about the same time
  __shared__ float wmax[4];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    atomicMax(reinterpret_cast<unsigned *>(pp.scales + 3 + t), __float_as_uint(m));
  }
}

// Q and K codes: 8 values per thread per step; block (0, 0) also publishes
// the three scales
__global__ __launch_bounds__(256) void attn_fp8_pack_qk_kernel(PackParams pp) {
  const int t = blockIdx.y;  // 0: q, 1: k
  const uint16_t *x = pp.x[t];
  uint8_t *y = t == 0 ? pp.q8 : pp.k8;
  const float inv = ldexpf(1.0f, -pow2_exp(pp.scales[3 + t]));
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < 3)
    pp.scales[threadIdx.x] = ldexpf(1.0f, pow2_exp(pp.scales[3 + threadIdx.x]));
  const long long n8 = pp.n[t] / 8;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
       i += (long long)gridDim.x * blockDim.x) {
    const bf16x8 v = __builtin_nontemporal_load((const bf16x8 *)(x + 8 * i));
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32((float)v[0] * inv, (float)v[1] * inv, 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32((float)v[2] * inv, (float)v[3] * inv, lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32((float)v[4] * inv, (float)v[5] * inv, 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32((float)v[6] * inv, (float)v[7] * inv, hi, true);
    typedef int i32x2 __attribute__((ext_vector_type(2)));
    __builtin_nontemporal_store(i32x2{lo, hi}, (i32x2 *)(y + 8 * i));
  }
}

// V^T codes: one workgroup per (b, kvh, 64-key tile); the tile's bf16 rows go
// through LDS and come out as D rows of 64 permuted key bytes.
template <int D>
__global__ __launch_bounds__(256) void attn_fp8_pack_vt_kernel(PackParams pp) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kBN8][D + 8];
  const int tiles = pp.Np / kBN8;
  const int tix = blockIdx.x % tiles;
  const int bk = blockIdx.x / tiles;  // b * Hkv + kvh
  const int j0 = tix * kBN8;
  const uint16_t *src = pp.x[2] + (size_t)bk * pp.N * D;
  const float inv = ldexpf(1.0f, -pow2_exp(pp.scales[5]));
  // load: 64 rows x D bf16, 8 values per thread per step, rows past N as 0
  for (int c = threadIdx.x; c < kBN8 * D / 8; c += blockDim.x) {
    const int r = c / (D / 8), col = 8 * (c % (D / 8));
    u32x4 v = u32x4{};
    if (j0 + r < pp.N) v = __builtin_nontemporal_load((const u32x4 *)(src + (size_t)(j0 + r) * D + col));
    *(u32x4 *)&tile[r][col] = v;
  }
  __syncthreads();
  // store: row d of V^T, 16 positions p = 16 c16 .. per thread per step
  uint8_t *dst = pp.vt8 + (size_t)bk * D * pp.Np + j0;
  for (int c = threadIdx.x; c < D * 4; c += blockDim.x) {
    const int d = c / 4, p0 = 16 * (c % 4);
    int w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float f[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int p = p0 + 4 * q + e;
        const int key = key_of(p >> 5, p & 31);
        f[e] = __uint_as_float((unsigned)tile[key][d] << 16) * inv;  // bf16 -> fp32, exact
      }
      int x = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
      w[q] = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], x, true);
    }
    __builtin_nontemporal_store(i32x4{w[0], w[1], w[2], w[3]}, (i32x4 *)(dst + (size_t)d * pp.Np + p0));
  }
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
struct F8Params {
  const uint8_t *q, *k, *vt;
  const float *scales;
  uint16_t *o;
  float *lse;
  int B, Hq, Hkv, N, Np;
  int G, groups, nq, total, nkt;
  float cs;      // |scale| * log2(e) (times s_q s_k in the kernel)
  int neg;       // scale < 0: q codes are negated on load (sign bit, exact)
  int causal, window;
};

template <int D>
struct F8Geo {
  static constexpr int kKB = D / 64;           // 64-wide k blocks of S
  static constexpr int kDB = D / 32;           // 32-row d blocks of O^T
  static constexpr int kKStride = D + 16;      // K tile row (bytes)
  static constexpr int kVStride = kBN8 + 16;   // V^T tile row (bytes)
  static constexpr int kKTile = kBN8 * kKStride;
  static constexpr int kVTile = D * kVStride;
  static constexpr int kSet = kKTile + kVTile;
};

template <int D, int NW>
struct F8Stage {
  // 16-byte chunks of K (64 rows x D bytes) and of V^T (D rows x 64 bytes):
  // D * 64 / 16 of each, kN per thread (chunk n * NW * 64 + tid)
  static constexpr int kChunks = D * kBN8 / 16;
  static constexpr int kN = (kChunks + NW * 64 - 1) / (NW * 64);
  i32x4 k[kN], v[kN];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                       int j0, int Np, int tid) {
#pragma unroll
    for (int n = 0; n < kN; ++n) {
      const int ci = n * NW * 64 + tid;
      if (ci < kChunks) {
        k[n] = __builtin_amdgcn_raw_buffer_load_b128(rk, j0 * D + ci * 16, 0, 0);
        const int d = ci / 4, c = ci % 4;
        v[n] = __builtin_amdgcn_raw_buffer_load_b128(rv, d * Np + j0 + c * 16, 0, 0);
      }
    }
  }
  __device__ __forceinline__ void store(lchar *set, int tid) const {
    using g = F8Geo<D>;
#pragma unroll
    for (int n = 0; n < kN; ++n) {
      const int ci = n * NW * 64 + tid;
      if (ci < kChunks) {
        const int r = ci / (D / 16), c = ci % (D / 16);
        *(lds_i32x4_t *)(set + r * g::kKStride + c * 16) = k[n];
        const int d = ci / 4, cv = ci % 4;
        *(lds_i32x4_t *)(set + g::kKTile + d * g::kVStride + cv * 16) = v[n];
      }
    }
  }
};

template <int D, int NW, int P>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 3 : 2) void attn_fwd_fp8_kernel(F8Params prm) {
  using g = F8Geo<D>;
  constexpr int kRows = 32 * NW / P;
  __shared__ __attribute__((aligned(1024))) char smem[2 * g::kSet];
  lchar *const set0 = (lchar *)smem;
  lchar *const set1 = (lchar *)smem + g::kSet;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const Task tk = make_task<P, kRows, kBN8>(prm, wave);
  const int N = prm.N;
  const float s_q = prm.scales[0], s_k = prm.scales[1], s_v = prm.scales[2];
  float c = prm.cs * s_q * s_k;
  c = c < FLT_MIN ? FLT_MIN : c;

  const __amdgpu_buffer_rsrc_t rs_k = make_rsrc(prm.k + tk.kv_slice * D, (uint32_t)N * D);
  const __amdgpu_buffer_rsrc_t rs_v =
      make_rsrc(prm.vt + (size_t)(tk.kv_slice / N) * D * prm.Np, (uint32_t)D * prm.Np);

  // Q^T operand: row qw0 + l32, bytes 64 kb + 32 hh .. + 31
  const int row = tk.qw0 + l32;
  i32x8 qf[g::kKB];
#pragma unroll
  for (int kb = 0; kb < g::kKB; ++kb) {
    i32x8 v = i32x8{};
    if (row < N) {
      const uint8_t *p = prm.q + (tk.q_slice + row) * D + 64 * kb + 32 * hh;
      const i32x4 a = *(const i32x4 *)p, b = *(const i32x4 *)(p + 16);
      v = i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
      if (prm.neg) v ^= (int)0x80808080u;
    }
    qf[kb] = v;
    settle(__builtin_shufflevector(v, v, 0, 1, 2, 3));
    settle(__builtin_shufflevector(v, v, 4, 5, 6, 7));
  }

  const int k_lane = l32 * g::kKStride + 32 * hh;
  const int v_lane = l32 * g::kVStride + 32 * hh;
  f32x16 oacc[g::kDB];
#pragma unroll
  for (int i = 0; i < g::kDB; ++i) oacc[i] = f32x16{};
  float m2 = -1e30f, lsum = 0.0f;

  // visible keys of this lane's row: lo < key <= hi
  const int m_hi = prm.causal ? min(row, N - 1) : N - 1;
  const int m_lo = prm.window > 0 ? row - prm.window : -1;

  F8Stage<D, NW> stage;
  if (tk.wg_lo < tk.wg_hi) {
    stage.load(rs_k, rs_v, tk.wg_lo * kBN8, prm.Np, tid);
    stage.store(set0, tid);
  }
  __syncthreads();

  auto compute = [&](int t, const lchar *set) {
    const int j0 = t * kBN8;
    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
      for (int kb = 0; kb < g::kKB; ++kb) {
        const lchar *p = set + k_lane + rb * 32 * g::kKStride + 64 * kb;
        const i32x4 a = *(const lds_i32x4_t *)p, b = *(const lds_i32x4_t *)(p + 16);
        const i32x8 kf = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        s[rb] = mfma8(kf, qf[kb], s[rb]);
      }
    }
    // mask: register r of block rb holds key j0 + 32 rb + 8 (r / 4) + 4 hh + r % 4
    const bool need_mask = edge_tile(prm.causal, prm.window, j0, kBN8, tk.qw0, N);
    if (need_mask) {
      const int kb0 = j0 + 4 * hh;
      const unsigned span = (unsigned)max(m_hi - m_lo, 0);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb0 + 32 * rb + 8 * (r >> 2) + (r & 3);
          s[rb][r] = (unsigned)(key - m_lo - 1) < span ? s[rb][r] : -INFINITY;
        }
      }
    }
    // tile max (scaled log2 units); the reference max moves lazily (kTau8)
    float mx = s[0][0];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[rb][r]);
    }
    const float mt = wave_max_pair(mx) * c;
    const bool move = __builtin_amdgcn_ballot_w64(mt > m2 + kTau8) != 0;
    const float mnew = move ? fmaxf(m2, mt) : m2;
    const float alpha = __builtin_amdgcn_exp2f(m2 - mnew);
    m2 = mnew;
    if (move) {
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < g::kDB; ++db) oacc[db] *= alpha;
    }
    const float off = kPShift - mnew;
    float part = 0.0f;
    int pw[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int b = 4 * w + e;  // byte b of the operand: block b / 16, register b % 16
        p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b >> 4][b & 15], c, off));
        part += p[e];
      }
      const int x = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
      pw[w] = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], x, true);
    }
    lsum += part;
    const i32x8 pf = {pw[0], pw[1], pw[2], pw[3], pw[4], pw[5], pw[6], pw[7]};
#pragma unroll
    for (int db = 0; db < g::kDB; ++db) {
      const lchar *p = set + g::kKTile + v_lane + db * 32 * g::kVStride;
      const i32x4 a = *(const lds_i32x4_t *)p, b = *(const lds_i32x4_t *)(p + 16);
      const i32x8 vf = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
      oacc[db] = mfma8(vf, pf, oacc[db]);
    }
  };

  auto step = [&](int t, const lchar *cur, lchar *next) {
    const bool more = t + 1 < tk.wg_hi;
    if (more) stage.load(rs_k, rs_v, (t + 1) * kBN8, prm.Np, tid);
    if (t >= tk.w_lo && t < tk.w_hi) compute(t, cur);
    if (more) stage.store(next, tid);
    __syncthreads();
  };
  for (int t = tk.wg_lo; t < tk.wg_hi; t += 2) {
    step(t, set0, set1);
    if (t + 1 < tk.wg_hi) step(t + 1, set1, set0);
  }

  const float ltot = wave_sum_pair(lsum);
  if (row >= N) return;
  store_rows<D>(prm.o + tk.q_slice * D, row, hh, oacc, s_v / ltot);
  if (hh == 0) prm.lse[tk.q_slice + row] = (m2 - kPShift + __builtin_amdgcn_logf(ltot)) * kLn2;
}

template <int D, int P>
hipError_t launch_fp8_t(const Fp8Problem &p, hipStream_t stream) {
  constexpr int NW = kF8Waves;
  constexpr int kRows = 32 * NW / P;
  F8Params prm{};
  prm.q = static_cast<const uint8_t *>(p.q8);
  prm.k = static_cast<const uint8_t *>(p.k8);
  prm.vt = static_cast<const uint8_t *>(p.vt8);
  prm.scales = p.scales;
  prm.o = static_cast<uint16_t *>(p.o);
  prm.lse = p.lse;
  prm.B = p.B; prm.Hq = p.Hq; prm.Hkv = p.Hkv; prm.N = p.N;
  prm.Np = (p.N + kBN8 - 1) / kBN8 * kBN8;
  prm.G = p.Hq / p.Hkv;
  prm.groups = p.Hq / P;
  prm.nq = (p.N + kRows - 1) / kRows;
  const long long total = (long long)p.B * prm.groups * prm.nq;
  if (total > 0x7fffffffLL) return hipErrorInvalidValue;
  prm.total = (int)total;
  prm.nkt = (p.N + kBN8 - 1) / kBN8;
  prm.cs = std::fabs(p.scale) * kLog2e;
  prm.neg = p.scale < 0.0f ? 1 : 0;
  prm.causal = p.causal;
  prm.window = p.window;
  void *args[] = {&prm};
  return hipLaunchKernel(reinterpret_cast<const void *>(&attn_fwd_fp8_kernel<D, NW, P>),
                         dim3(prm.total), dim3(NW * 64), args, 0, stream);
}

template <int D>
hipError_t launch_fp8_d(const Fp8Problem &p, hipStream_t stream) {
  const int G = p.Hq / p.Hkv;
  if (kF8Waves >= 8 && G % 8 == 0) return launch_fp8_t<D, kF8Waves >= 8 ? 8 : 4>(p, stream);
  if (G % 4 == 0) return launch_fp8_t<D, 4>(p, stream);
  if (G % 2 == 0) return launch_fp8_t<D, 2>(p, stream);
  return launch_fp8_t<D, 1>(p, stream);
}

template <int D>
hipError_t launch_pack_d(const Fp8Pack &p, hipStream_t stream) {
  PackParams pp{};
  pp.x[0] = static_cast<const uint16_t *>(p.q);
  pp.x[1] = static_cast<const uint16_t *>(p.k);
  pp.x[2] = static_cast<const uint16_t *>(p.v);
  pp.q8 = static_cast<uint8_t *>(p.q8);
  pp.k8 = static_cast<uint8_t *>(p.k8);
  pp.vt8 = static_cast<uint8_t *>(p.vt8);
  pp.scales = p.scales;
  pp.n[0] = (long long)p.B * p.Hq * p.N * D;
  pp.n[1] = (long long)p.B * p.Hkv * p.N * D;
  pp.n[2] = pp.n[1];
  pp.B = p.B; pp.Hkv = p.Hkv; pp.N = p.N;
  pp.Np = (p.N + kBN8 - 1) / kBN8 * kBN8;
  void *args[] = {&pp};
  void *clear_args[] = {&pp.scales};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&attn_fp8_clear_kernel), dim3(1),
                                 dim3(64), clear_args, 0, stream);
  if (e != hipSuccess) return e;
  e = hipLaunchKernel(reinterpret_cast<const void *>(&attn_fp8_amax_kernel), dim3(512, 3),
                      dim3(256), args, 0, stream);
  if (e != hipSuccess) return e;
  e = hipLaunchKernel(reinterpret_cast<const void *>(&attn_fp8_pack_qk_kernel), dim3(2048, 2),
                      dim3(256), args, 0, stream);
  if (e != hipSuccess) return e;
  const long long wgs = (long long)p.B * p.Hkv * (pp.Np / kBN8);
  if (wgs > 0x7fffffffLL) return hipErrorInvalidValue;
  return hipLaunchKernel(reinterpret_cast<const void *>(&attn_fp8_pack_vt_kernel<D>),
                         dim3((unsigned)wgs), dim3(256), args, 0, stream);
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8Problem &p, hipStream_t stream) {
  return p.d == 128 ? launch_fp8_d<128>(p, stream) : launch_fp8_d<64>(p, stream);
}

hipError_t launch_fp8_pack(const Fp8Pack &p, hipStream_t stream) {
  return p.d == 128 ? launch_pack_d<128>(p, stream) : launch_pack_d<64>(p, stream);
}

}  // namespace attn
