// Device-side building blocks shared by the gfx950 attention kernels.
// Private to the library; included by the .hip sources only.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace attn {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((vector_size(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8_t;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4_t;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4_t;
typedef __attribute__((address_space(3))) float lds_f32_t;
typedef char __attribute__((address_space(3))) lchar;

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kBufferFlags = 0x00020000;  // gfx9 buffer descriptor word 3

// LDS row strides for a tile of rows of D bf16 values.  Rows read with
// ds_read_b128 (16 lanes, 16 consecutive rows per phase) are padded by 16
// bytes, so those rows start 4 banks apart; rows read with the transposing
// ds_read_b64_tr_b16 (4 consecutive rows per 16-lane group) are padded by 64
// bytes, so they start 16 banks apart.  Fragment addresses are then a
// per-lane base plus a compile-time offset.
template <int D>
struct Stride {
  static constexpr int kRowB = D * 2;       // bytes per row in HBM
  static constexpr int kCh = kRowB / 16;    // 16-byte chunks per row
  static constexpr int kB128 = kRowB + 16;  // LDS stride for b128 reads
  static constexpr int kTr = kRowB + 64;    // LDS stride for transposed reads
  static constexpr int kKSteps = D / 16;    // 16-wide k-steps over d
  static constexpr int kDB = D / 32;        // 32-wide blocks of d
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

__device__ __forceinline__ float wave_max_pair(float x) {
  // max of this lane and lane ^ 32
  auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float wave_sum_pair(float x) {
  auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// Waits here for the load that produced x.  A value loaded before a loop
// and first read inside it otherwise makes the compiler wait for every
// outstanding load at that read on each iteration, including the loads of
// the next tile issued just before.
template <class T>
__device__ __forceinline__ void settle(const T &x) {
  asm volatile("" ::"v"(x));
}

// Per-lane byte offset of a b128 MFMA fragment in a tile of stride STRIDE:
// row lane % 32, d = 16 * kk + 8 * (lane / 32) .. + 7 for k-step kk (the
// k-step's 32 bytes are added by b128_frag).
template <int STRIDE>
__device__ __forceinline__ int b128_lane_off(int lane) {
  return (lane & 31) * STRIDE + (lane >> 5) * 16;
}
// Fragment (k-step kk, 32-row block rb) from a tile base already offset by
// b128_lane_off.
template <int STRIDE>
__device__ __forceinline__ bf16x8 b128_frag(const lchar *base, int kk, int rb) {
  return *(const lds_bf16x8_t *)(base + rb * 32 * STRIDE + kk * 32);
}

// Per-lane byte offset of a transposed fragment in a tile of stride STRIDE:
// tile row 4 * (lane / 32) + (lane & 15) / 4 (+ the fragment's row base),
// column 16 * ((lane >> 4) & 1) + 4 * (lane & 3) .. + 3.
template <int STRIDE>
__device__ __forceinline__ int tr_lane_off(int lane) {
  return (4 * (lane >> 5) + ((lane & 15) >> 2)) * STRIDE + (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
}
// Transposed fragment: A operand rows = columns 32 * db .. of the tile, k =
// the 16 tile rows 32 * rb + 16 * tt .., as two ds_read_b64_tr_b16 of 4 rows
// each (in each 16-lane group, lane 4j + c supplies the address of 4
// consecutive columns of row j and lane i receives column i).  The k order
// matches the register order of an MFMA accumulator used as the B operand.
template <int STRIDE>
__device__ __forceinline__ bf16x8 tr_frag(const lchar *base, int db, int rb, int tt) {
  const lchar *p = base + (32 * rb + 16 * tt) * STRIDE + db * 64;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)p);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(p + 8 * STRIDE));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, both);
}

// Launch order of the query-tiled kernels (the forwards and the backward's
// dQ kernel): a workgroup serves query-tile rank qrank of head group
// hgb = batch * groups + head group, P heads per workgroup (wave w serves
// head w % P on rows (w / P) * 32 ..); causal ranks run heaviest first
// (rank 0 is the last row tile).  Prm must provide groups, nq, causal, G.
struct TileSlot {
  int b, head, kvh;
  int wg_r0;  // first query row of the workgroup
  int qw0;    // first query row of this wave
};

template <int P, int kRows, class Prm>
__device__ __forceinline__ TileSlot tile_slot(const Prm &prm, int wave, int qrank, int hgb) {
  TileSlot t;
  const int hg = hgb % prm.groups;
  t.b = hgb / prm.groups;
  const int qi = prm.causal ? (prm.nq - 1 - qrank) : qrank;  // heaviest tiles first
  t.head = hg * P + (wave % P);
  t.kvh = __builtin_amdgcn_readfirstlane((hg * P) / prm.G);  // P divides G
  t.wg_r0 = qi * kRows;
  t.qw0 = t.wg_r0 + (wave / P) * 32;
  return t;
}

// One workgroup per query tile: hardware workgroup id -> (qrank, hgb), the
// logical id xcd_remap(id) = hgb * nq + qrank, so the tiles of one head run
// behind one L2.  Prm must provide total and nq.
template <class Prm>
__device__ __forceinline__ void dense_slot(const Prm &prm, int id, int &qrank, int &hgb) {
  const int logical = xcd_remap(id, prm.total);
  qrank = logical % prm.nq;
  hgb = logical / prm.nq;
}

// Keys [lo, hi) that query rows [r0, r1) of an N-row sequence may see under
// the causal mask and the causal window (row i sees i - window < j <= i).
__device__ __forceinline__ void causal_window_keys(int causal, int window, int r0, int r1, int N,
                                                   int &lo, int &hi) {
  hi = causal ? r1 : N;
  lo = window > 0 ? max(0, r0 - window + 1) : 0;
}

// Whether the 32 query rows from qw0 hold a pair of keys [j0, j0 + kbn)
// that is masked (diagonal, window edge) or past N: only such tiles run
// the mask.
__device__ __forceinline__ bool edge_tile(int causal, int window, int j0, int kbn, int qw0,
                                          int N) {
  return (causal && j0 + kbn - 1 > qw0) || (window > 0 && j0 <= qw0 + 31 - window) ||
         (j0 + kbn > N);
}

// The dense task of a query-tiled workgroup with KBN-key tiles.
// Prm must provide total, nq, groups, causal, window, G, nkt, N, Hq, Hkv.
struct Task {
  int b, head, kvh;
  int qw0;             // first query row of this wave
  int wg_lo, wg_hi;    // key tiles any row of the workgroup sees
  int w_lo, w_hi;      // key tiles any row of this wave sees
  size_t q_slice;      // (b * Hq + head) * N: first row of the Q / O slice
  size_t kv_slice;     // (b * Hkv + kvh) * N: first row of the K / V slice
};

template <int P, int kRows, int KBN, class Prm>
__device__ __forceinline__ Task make_task(const Prm &prm, int wave) {
  int qrank, hgb;
  dense_slot(prm, blockIdx.x, qrank, hgb);
  const TileSlot sl = tile_slot<P, kRows>(prm, wave, qrank, hgb);
  Task tk;
  tk.b = sl.b;
  tk.head = sl.head;
  tk.kvh = sl.kvh;
  tk.qw0 = sl.qw0;
  const int N = prm.N;
  auto tile_range = [&](int r0, int r1, int &lo, int &hi) {  // rows [r0, r1)
    int klo, khi;
    causal_window_keys(prm.causal, prm.window, r0, r1, N, klo, khi);
    lo = klo / KBN;
    hi = min(prm.nkt, (khi + KBN - 1) / KBN);
  };
  tile_range(sl.wg_r0, min(N, sl.wg_r0 + kRows), tk.wg_lo, tk.wg_hi);
  if (tk.qw0 < N) {
    tile_range(tk.qw0, min(N, tk.qw0 + 32), tk.w_lo, tk.w_hi);
  } else {
    tk.w_lo = tk.w_hi = 0;  // rows past the end: this wave only helps load tiles
  }
  tk.kv_slice = (size_t)(tk.b * prm.Hkv + tk.kvh) * N;
  tk.q_slice = (size_t)(tk.b * prm.Hq + tk.head) * N;
  return tk;
}

// The 8 d values d0 .. d0 + 7 of row `row` of a [rows][D] bf16 slice as an
// MFMA operand fragment; zero past the last row, sign-flipped when neg
// (exact in bf16).
template <int D>
__device__ __forceinline__ bf16x8 row_frag(const uint16_t *slice, int row, int N, int d0, bool neg) {
  bf16x8 f = row < N ? *(const bf16x8 *)(slice + (size_t)row * D + d0) : bf16x8{};
  if (neg) {
    u32x4 t = __builtin_bit_cast(u32x4, f);
    t ^= 0x80008000u;
    f = __builtin_bit_cast(bf16x8, t);
  }
  return f;
}

// Stores one lane's share of a transposed 32-row accumulator block set:
// acc[db] holds columns 32 * db + 8 * (r / 4) + 4 * (lane / 32) + r % 4 of
// row `row` (= this lane's row), scaled by mul, as bf16 (RNE).
template <int D>
__device__ __forceinline__ void store_rows(uint16_t *slice, int row, int hh,
                                           const f32x16 (&acc)[Stride<D>::kDB], float mul) {
  uint16_t *op = slice + (size_t)row * D + 4 * hh;
#pragma unroll
  for (int db = 0; db < Stride<D>::kDB; ++db) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = (__bf16)(acc[db][4 * i + j] * mul);
      *(bf16x4 *)(op + 32 * db + 8 * i) = w;
    }
  }
}

}  // namespace dev
}  // namespace attn
