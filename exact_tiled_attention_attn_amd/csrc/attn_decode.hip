// gfx950 (MI355X, CDNA4) decode attention over a paged KV cache, split over
// the keys.
//
// What is computed: "Efficient attention: long context and sub-quadratic
// variants", section "FlashAttention: exact attention, IO-aware", describes
// PagedAttention: the KV cache sits in fixed-size pages, each sequence has a
// page table, attention gathers K and V through it, and the result is the
// exact attention.  The T newest tokens of sequence b are the queries; query
// t sits at position L_b - T + t and sees the cached keys j <= that position
// (and j > pos - window with a window); query head h reads KV head
// h / (Hq / Hkv).
//
// Schedule (split-KV): one single-wave workgroup per (sequence, KV head,
// key range of `chunk` keys, block of 32 columns).  The G query heads x T
// tokens of the KV group are the MFMA columns, 32 per wave, so every cached
// K/V byte is read from HBM once for all the heads that share it; with more
// than 32 columns (multi-query attention at real head counts, several new
// tokens) the column blocks of one key range run on one XCD, one after the
// other in dispatch order, and all but the first find the K/V tiles in that
// XCD's L2.  32-key tiles are gathered
// through the page table (two 16-row groups per tile, each inside one page)
// and staged two tiles ahead through registers into the wave's LDS tile.
// Per tile: S^T = K Q^T (8 MFMA), running max / sum per column, O^T += V^T
// P^T (8 MFMA, V^T by transposing LDS reads).  The split writes its
// normalised partial (O_s, lse_s); attn_decode_merge_kernel combines the
// splits with lse = ln sum_s exp(lse_s), O = sum_s exp(lse_s - lse) O_s,
// which is the running softmax's rescaling applied once per split.
//
// The kernel is bound by HBM: per cached token it reads 2 x d x 2 bytes and
// does 4 d G T FLOPs.  When a call's K/V may exceed the last-level cache
// the K/V loads are nontemporal (they stream through the caches); smaller
// calls use ordinary loads, whose lines can stay cached between calls.

#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstdint>

#include <mutex>

#include "attn.h"
#include "attn_device.h"
#include "attn_internal.h"

namespace attn {
namespace {

using namespace dev;

constexpr int kKeys = 32;       // keys per tile
constexpr int kMaxEntries = 64;  // page-table entries per split (one per lane)
constexpr float kTau = 8.0f;        // lazy-rescale threshold of the multi-column kernel, log2 units
constexpr double kLastLevelCacheBytes = 256.0 * 1024 * 1024;  // MI355X Infinity Cache

struct DecParams {
  const uint16_t *q, *kc, *vc;  // q [B][Hq][T][D]; caches [pages][PS][Hkv][D]
  const int *table, *lens;      // [B][max_pages], [B]
  uint16_t *o;                  // [B][Hq][T][D]
  float *lse;                   // [B][Hq][T]
  float *part_o;                // [B][Hkv][nsplit][ncols][D]
  float *part_lse;              // [B][Hkv][nsplit][ncols]
  int B, Hq, Hkv, G, T, ncols;  // ncols = G * T
  int ncb, nwork;               // 32-column blocks; (sequence, split, KV head) items
  int ps, ps_shift;             // page size (power of two)
  int num_pages, max_pages;
  int nsplit, chunk;            // keys per split: multiple of unit
  int unit;                     // max(32, ps): splits start on a page and a tile
  float c;                      // |scale| * log2(e), at least FLT_MIN
  int neg;                      // scale < 0: q is negated on load
  int window;                   // 0: none
};

template <int D>
struct DecTile {
  using st = Stride<D>;
  static constexpr int kKB = kKeys * st::kB128;  // K tile, b128 stride
  static constexpr int kVB = kKeys * st::kTr;    // V tile, transposed-read stride
  static constexpr int kSet = kKB + kVB;
  static constexpr int kLoads = kKeys * st::kCh / 64;  // b128 per lane per tensor
  static constexpr int kRowsPerLoad = 64 / st::kCh;
};

// Buffer descriptor over the 16 cached rows starting at token j (a multiple
// of 16, so the rows lie in one page) of KV head kvh; rows at or past the
// sequence length, and every row of an out-of-range page index, read as 0.
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t group_rsrc(const uint16_t *cache,
                                                           const DecParams &prm, int page,
                                                           int j, int L, int kvh) {
  const int valid = min(max(L - j, 0), 16);
  const bool ok = valid > 0 && page >= 0 && page < prm.num_pages;
  const size_t row = (size_t)page * prm.ps + (j & (prm.ps - 1));
  const uint16_t *base = cache + (ok ? (row * prm.Hkv + kvh) * D : 0);
  const uint32_t stride = (uint32_t)prm.Hkv * D * 2;
  const uint32_t bytes = ok ? (uint32_t)(valid - 1) * stride + D * 2 : 0;
  return make_rsrc(base, bytes);
}

// Cache policy of the K/V loads: 0, or 2 (nontemporal: stream through the
// caches without keeping the lines).
template <int D, int kPol>
struct DecStage {
  using tl = DecTile<D>;
  u32x4 k[tl::kLoads], v[tl::kLoads];

  // Tile of keys j0 .. j0 + 31; lane loads row 4n + lane / 16 (n-th load),
  // 16-byte chunk lane % 16 of it (for D = 128).
  __device__ __forceinline__ void load(const DecParams &prm, int page0, int page1, int j0, int L,
                                       int kvh, int lane) {
    const __amdgpu_buffer_rsrc_t k0 = group_rsrc<D>(prm.kc, prm, page0, j0, L, kvh);
    const __amdgpu_buffer_rsrc_t k1 = group_rsrc<D>(prm.kc, prm, page1, j0 + 16, L, kvh);
    const __amdgpu_buffer_rsrc_t v0 = group_rsrc<D>(prm.vc, prm, page0, j0, L, kvh);
    const __amdgpu_buffer_rsrc_t v1 = group_rsrc<D>(prm.vc, prm, page1, j0 + 16, L, kvh);
    const uint32_t stride = (uint32_t)prm.Hkv * D * 2;
    const int r_lane = lane / Stride<D>::kCh, ch = lane % Stride<D>::kCh;
#pragma unroll
    for (int n = 0; n < tl::kLoads; ++n) {
      const int r = n * tl::kRowsPerLoad + r_lane;  // tile row 0 .. 31
      const uint32_t off = (uint32_t)(r & 15) * stride + ch * 16;
      const bool hi = n * tl::kRowsPerLoad >= 16;   // compile-time per n
      k[n] = __builtin_amdgcn_raw_buffer_load_b128(hi ? k1 : k0, off, 0, kPol);
      v[n] = __builtin_amdgcn_raw_buffer_load_b128(hi ? v1 : v0, off, 0, kPol);
    }
  }
  __device__ __forceinline__ void store(lchar *set, int lane) const {
    const int r_lane = lane / Stride<D>::kCh, ch = lane % Stride<D>::kCh;
#pragma unroll
    for (int n = 0; n < tl::kLoads; ++n) {
      const int r = n * tl::kRowsPerLoad + r_lane;
      *(lds_u32x4_t *)(set + r * Stride<D>::kB128 + ch * 16) = k[n];
      *(lds_u32x4_t *)(set + tl::kKB + r * Stride<D>::kTr + ch * 16) = v[n];
    }
  }
};

template <int D, int kPol>
__global__ __launch_bounds__(64) void attn_decode_split_kernel(DecParams prm) {
  using st = Stride<D>;
  using tl = DecTile<D>;
  __shared__ __attribute__((aligned(1024))) char smem[tl::kSet];

  const int lane = threadIdx.x;
  const int l32 = lane & 31, hh = lane >> 5;
  // work item w = (b * nsplit + split) * Hkv + kvh: the Hkv workgroups that
  // read the same cache pages (token rows hold every KV head) run together,
  // so each page is streamed from HBM in one pass rather than in Hkv
  // scattered 256-byte pieces.  Column block cb of item w is workgroup
  // 8 (ncb (w / 8) + cb) + w % 8: the same XCD (workgroups go to the 8 XCDs
  // in turn) and 8 ids after block cb - 1.  With one block, w = blockIdx.x.
  const int u = blockIdx.x;
  const int cb = (u >> 3) % prm.ncb;
  const int w = ((u >> 3) / prm.ncb) * 8 + (u & 7);
  if (w >= prm.nwork) return;  // padding of the last group of 8 items
  const int kvh = w % prm.Hkv;
  const int bs = w / prm.Hkv;
  const int split = bs % prm.nsplit, b = bs / prm.nsplit;
  const int bk = b * prm.Hkv + kvh;
  const int L = prm.lens[b];
  const int T = prm.T;

  // this lane's column: query head kvh * G + g, token t
  const int col = 32 * cb + l32;
  const bool col_ok = col < prm.ncols;
  const int g = col_ok ? col / T : 0, t = col_ok ? col % T : 0;
  const int pos = L - T + t;                   // position of the query token
  const int m_lo = prm.window > 0 ? max(0, pos - prm.window + 1) : 0;
  const int m_span = col_ok && pos >= 0 ? pos - m_lo + 1 : 0;  // visible keys [m_lo, pos]

  // key range of this split: the splits tile the keys any column sees,
  // from the window start of the first query (rounded down to a page and a
  // tile) on
  const int lo_all = prm.window > 0 ? max(0, L - T - prm.window + 1) : 0;
  const int s_lo = (lo_all / prm.unit) * prm.unit + split * prm.chunk;
  const int k_begin = max(s_lo, lo_all & ~(kKeys - 1));
  const int k_end = min(s_lo + prm.chunk, L);
  const int ntiles = k_end > k_begin ? (k_end - k_begin + kKeys - 1) / kKeys : 0;

  // page-table entries of the split: lane i holds entry s_lo / ps + i
  const int e0 = s_lo >> prm.ps_shift;
  int entry = -1;
  if (e0 + lane < prm.max_pages && lane < kMaxEntries)
    entry = prm.table[(size_t)b * prm.max_pages + e0 + lane];
  auto page_of = [&](int j) {  // page holding token j of this split
    return __builtin_amdgcn_readlane(entry, (j >> prm.ps_shift) - e0);
  };

  // Q^T operand: column col, d = 16 kk + 8 hh ..
  const size_t q_row = ((size_t)(b * prm.Hq + kvh * prm.G + g) * T + t);
  bf16x8 qf[st::kKSteps];
#pragma unroll
  for (int kk = 0; kk < st::kKSteps; ++kk) {
    qf[kk] = row_frag<D>(prm.q + q_row * D, 0, col_ok ? 1 : 0, 16 * kk + 8 * hh, prm.neg);
    settle(qf[kk]);
  }
  settle(entry);

  f32x16 oacc[st::kDB];
#pragma unroll
  for (int i = 0; i < st::kDB; ++i) oacc[i] = f32x16{};
  float m2 = -1e30f, lsum = 0.0f, lrnd = 0.0f;
  const float c = prm.c;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  const int kb_lane = b128_lane_off<st::kB128>(lane);
  const int vt_lane = tr_lane_off<st::kTr>(lane);

  auto compute = [&](int j0, const lchar *set) {
    // S^T: register r holds key j0 + 8 (r / 4) + 4 hh + r % 4 of this column
    f32x16 s = f32x16{};
#pragma unroll
    for (int kk = 0; kk < st::kKSteps; ++kk)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b128_frag<st::kB128>(set + kb_lane, kk, 0),
                                                  qf[kk], s, 0, 0, 0);
    // every valid column sees the whole tile when it starts at or after the
    // last column's window start and ends at or before the first column's
    // position
    const bool need_mask = (prm.window > 0 && j0 < L - prm.window) || j0 + kKeys - 1 > L - T;
    if (need_mask) {
      const int base = j0 + 4 * hh - m_lo;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        s[r] = (unsigned)(base + 8 * (r >> 2) + (r & 3)) < (unsigned)m_span ? s[r] : -INFINITY;
    }
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = wave_max_pair(mx) * c;  // scaled, log2 units; -inf if nothing visible
    const float mnew = fmaxf(m2, mx);
    const float alpha = __builtin_amdgcn_exp2f(m2 - mnew);
    m2 = mnew;
    bf16x8 pf[2];
    float ps = 0.0f, pr = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -mnew));
      ps += p;
      pf[r >> 3][r & 7] = (__bf16)p;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bf16x2 pair = {pf[i >> 2][2 * (i & 3)], pf[i >> 2][2 * (i & 3) + 1]};
      pr = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, pr, false);
    }
    lsum = lsum * alpha + wave_sum_pair(ps);
    lrnd = lrnd * alpha + wave_sum_pair(pr);
#pragma unroll
    for (int db = 0; db < st::kDB; ++db) {
      oacc[db] *= alpha;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            tr_frag<st::kTr>(set + tl::kKB + vt_lane, db, 0, tt), pf[tt], oacc[db], 0, 0, 0);
    }
  };

  // One LDS tile per wave: the wave's LDS instructions execute in order,
  // so the next tile's stores, issued after this tile's reads, cannot
  // overwrite data those reads still have to return.  Two tiles are in
  // flight in registers (sa, sb) while one is computed.
  lchar *const set = (lchar *)smem;
  DecStage<D, kPol> sa, sb;
  auto tile_j0 = [&](int i) { return k_begin + i * kKeys; };
  auto issue = [&](DecStage<D, kPol> &sg, int i) {
    const int j0 = tile_j0(i);
    sg.load(prm, page_of(j0), page_of(j0 + 16), j0, L, kvh, lane);
  };
  if (ntiles > 0) issue(sa, 0);
  if (ntiles > 1) issue(sb, 1);
  if (ntiles > 0) sa.store(set, lane);
  for (int i = 0; i < ntiles; i += 2) {
    // tile i is in LDS, tile i + 1 in sb; tile i + 2 loads into sa
    if (i + 2 < ntiles) issue(sa, i + 2);
    compute(tile_j0(i), set);
    if (i + 1 >= ntiles) break;
    sb.store(set, lane);
    if (i + 3 < ntiles) issue(sb, i + 3);
    compute(tile_j0(i + 1), set);
    if (i + 2 < ntiles) sa.store(set, lane);
  }

  // partial result of this split for the lane's column
  const bool any = lsum > 0.0f;
  const float lse_s = any ? (m2 + __log2f(lsum)) * kLn2 : -INFINITY;
  const float inv = any ? 1.0f / lrnd : 0.0f;
  if (col_ok) {
    const size_t slot = ((size_t)bk * prm.nsplit + split) * prm.ncols + col;
    float *po = prm.part_o + slot * D + 4 * hh;
#pragma unroll
    for (int db = 0; db < st::kDB; ++db) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = oacc[db][4 * i + j] * inv;
        *(f32x4 *)(po + 32 * db + 8 * i) = w;
      }
    }
    if (hh == 0) prm.part_lse[slot] = lse_s;
  }
}

// More than 32 columns per KV head (multi-query attention at real head
// counts, several new tokens): one workgroup of W waves per (sequence,
// split, KV head, group of W column blocks), wave w computing column block
// W g + w.  The waves share each K/V tile: every wave gathers 1 / W of its
// rows, the tile goes to one of two LDS sets, and a barrier per tile
// publishes it; the compute is the single-wave kernel's.
template <int D, int kPol, int W>
struct DecStageW {
  using tl = DecTile<D>;
  static constexpr int kM = tl::kLoads / W;  // loads per lane per tensor
  static_assert(kM * W == tl::kLoads, "W must divide the loads of a tile");
  u32x4 k[kM], v[kM];
  // load n = W m + wave of the single-wave kernel's order (rows
  // n * kRowsPerLoad + lane / kCh, 16-byte chunk lane % kCh)
  __device__ __forceinline__ void load(const DecParams &prm, int page0, int page1, int j0, int L,
                                       int kvh, int lane, int wave) {
    const __amdgpu_buffer_rsrc_t k0 = group_rsrc<D>(prm.kc, prm, page0, j0, L, kvh);
    const __amdgpu_buffer_rsrc_t k1 = group_rsrc<D>(prm.kc, prm, page1, j0 + 16, L, kvh);
    const __amdgpu_buffer_rsrc_t v0 = group_rsrc<D>(prm.vc, prm, page0, j0, L, kvh);
    const __amdgpu_buffer_rsrc_t v1 = group_rsrc<D>(prm.vc, prm, page1, j0 + 16, L, kvh);
    const uint32_t stride = (uint32_t)prm.Hkv * D * 2;
    const int r_lane = lane / Stride<D>::kCh, ch = lane % Stride<D>::kCh;
#pragma unroll
    for (int m = 0; m < kM; ++m) {
      const int n = W * m + wave;
      const int r = n * tl::kRowsPerLoad + r_lane;  // tile row 0 .. 31
      const uint32_t off = (uint32_t)(r & 15) * stride + ch * 16;
      const bool hi = n * tl::kRowsPerLoad >= 16;   // wave-uniform
      k[m] = __builtin_amdgcn_raw_buffer_load_b128(hi ? k1 : k0, off, 0, kPol);
      v[m] = __builtin_amdgcn_raw_buffer_load_b128(hi ? v1 : v0, off, 0, kPol);
    }
  }
  __device__ __forceinline__ void store(lchar *set, int lane, int wave) const {
    const int r_lane = lane / Stride<D>::kCh, ch = lane % Stride<D>::kCh;
#pragma unroll
    for (int m = 0; m < kM; ++m) {
      const int r = (W * m + wave) * tl::kRowsPerLoad + r_lane;
      *(lds_u32x4_t *)(set + r * Stride<D>::kB128 + ch * 16) = k[m];
      *(lds_u32x4_t *)(set + tl::kKB + r * Stride<D>::kTr + ch * 16) = v[m];
    }
  }
};

template <int D, int kPol, int W>
__global__ __launch_bounds__(64 * W) void attn_decode_split_mc_kernel(DecParams prm) {
  using st = Stride<D>;
  using tl = DecTile<D>;
  __shared__ __attribute__((aligned(1024))) char smem[2 * tl::kSet];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  // item w and group gi of its ceil(ncb / W) column-block groups: with more
  // than one group, group gi of item w is workgroup 8 (ngr (w / 8) + gi) + w % 8
  // (same XCD as the item's other groups, 8 ids apart)
  const int ngr = (prm.ncb + W - 1) / W;
  const int u = blockIdx.x;
  const int gi = ngr == 1 ? 0 : (u >> 3) % ngr;
  const int w = ngr == 1 ? u : ((u >> 3) / ngr) * 8 + (u & 7);
  if (w >= prm.nwork) return;  // padding of the last group of 8 items
  const int kvh = w % prm.Hkv;
  const int bs = w / prm.Hkv;
  const int split = bs % prm.nsplit, b = bs / prm.nsplit;
  const int bk = b * prm.Hkv + kvh;
  const int L = prm.lens[b];
  const int T = prm.T;

  const int col = 32 * (W * gi + wave) + l32;
  const bool col_ok = col < prm.ncols;
  const int g = col_ok ? col / T : 0, t = col_ok ? col % T : 0;
  const int pos = L - T + t;
  const int m_lo = prm.window > 0 ? max(0, pos - prm.window + 1) : 0;
  const int m_span = col_ok && pos >= 0 ? pos - m_lo + 1 : 0;

  const int lo_all = prm.window > 0 ? max(0, L - T - prm.window + 1) : 0;
  const int s_lo = (lo_all / prm.unit) * prm.unit + split * prm.chunk;
  const int k_begin = max(s_lo, lo_all & ~(kKeys - 1));
  const int k_end = min(s_lo + prm.chunk, L);
  const int ntiles = k_end > k_begin ? (k_end - k_begin + kKeys - 1) / kKeys : 0;

  const int e0 = s_lo >> prm.ps_shift;
  int entry = -1;
  if (e0 + lane < prm.max_pages && lane < kMaxEntries)
    entry = prm.table[(size_t)b * prm.max_pages + e0 + lane];
  auto page_of = [&](int j) { return __builtin_amdgcn_readlane(entry, (j >> prm.ps_shift) - e0); };

  const size_t q_row = ((size_t)(b * prm.Hq + kvh * prm.G + g) * T + t);
  bf16x8 qf[st::kKSteps];
#pragma unroll
  for (int kk = 0; kk < st::kKSteps; ++kk) {
    qf[kk] = row_frag<D>(prm.q + q_row * D, 0, col_ok ? 1 : 0, 16 * kk + 8 * hh, prm.neg);
    settle(qf[kk]);
  }
  settle(entry);

  f32x16 oacc[st::kDB];
#pragma unroll
  for (int i = 0; i < st::kDB; ++i) oacc[i] = f32x16{};
  float m2 = -1e30f, lsum = 0.0f, lrnd = 0.0f;
  const float c = prm.c;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  const int kb_lane = b128_lane_off<st::kB128>(lane);
  const int vt_lane = tr_lane_off<st::kTr>(lane);

  auto compute = [&](int j0, const lchar *set) {
    f32x16 s = f32x16{};
#pragma unroll
    for (int kk = 0; kk < st::kKSteps; ++kk)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b128_frag<st::kB128>(set + kb_lane, kk, 0),
                                                  qf[kk], s, 0, 0, 0);
    const bool need_mask = (prm.window > 0 && j0 < L - prm.window) || j0 + kKeys - 1 > L - T;
    if (need_mask) {
      const int base = j0 + 4 * hh - m_lo;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        s[r] = (unsigned)(base + 8 * (r >> 2) + (r & 3)) < (unsigned)m_span ? s[r] : -INFINITY;
    }
    // Row max as a max3 tree; the reference max m2 moves (and O, and the
    // lane's two partial sums, are rescaled) only when some column's tile
    // max exceeds it by more than 2^kTau: the weights stay below 2^kTau, and
    // O, l and l~ carry the same reference, so the result is unchanged up to
    // rounding.  The sums are per lane, in independent chains, and are
    // combined with the partner lane (the column's other 16 keys) at the end.
    const float q0 = fmaxf(fmaxf(s[0], s[1]), s[2]), q1 = fmaxf(fmaxf(s[3], s[4]), s[5]);
    const float q2 = fmaxf(fmaxf(s[6], s[7]), s[8]), q3 = fmaxf(fmaxf(s[9], s[10]), s[11]);
    const float q4 = fmaxf(fmaxf(s[12], s[13]), s[14]);
    const float mx = wave_max_pair(fmaxf(fmaxf(fmaxf(q0, q1), q2), fmaxf(fmaxf(q3, q4), s[15]))) * c;
    if (__builtin_amdgcn_ballot_w64(mx > m2 + kTau) != 0) {
      const float mnew = fmaxf(m2, mx);
      const float alpha = __builtin_amdgcn_exp2f(m2 - mnew);
      lsum *= alpha;
      lrnd *= alpha;
#pragma unroll
      for (int db = 0; db < st::kDB; ++db) oacc[db] *= alpha;
      m2 = mnew;
    }
    bf16x8 pf[2];
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -m2));
      pf[r >> 3][r & 7] = (__bf16)p[r];
    }
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x2 a = {pf[i >> 1][4 * (i & 1)], pf[i >> 1][4 * (i & 1) + 1]};
      const bf16x2 b2 = {pf[i >> 1][4 * (i & 1) + 2], pf[i >> 1][4 * (i & 1) + 3]};
      pr[i] = __builtin_amdgcn_fdot2_f32_bf16(b2, ones, __builtin_amdgcn_fdot2_f32_bf16(a, ones, 0.0f, false), false);
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) p[r] += p[r + 8];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] += p[r + 4];
    lsum += (p[0] + p[1]) + (p[2] + p[3]);
    lrnd += (pr[0] + pr[1]) + (pr[2] + pr[3]);
#pragma unroll
    for (int db = 0; db < st::kDB; ++db) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            tr_frag<st::kTr>(set + tl::kKB + vt_lane, db, 0, tt), pf[tt], oacc[db], 0, 0, 0);
    }
  };

  // Tile i sits in LDS set i % 2; while it is computed, tile i + 1 (loaded
  // a step earlier) goes to the other set and tile i + 2 starts loading.
  // One barrier per tile: a set is rewritten only after every wave has
  // passed the barrier that ends its computation.
  auto set_of = [&](int i) { return (lchar *)smem + (i & 1) * tl::kSet; };
  auto tile_j0 = [&](int i) { return k_begin + i * kKeys; };
  DecStageW<D, kPol, W> stage;
  auto issue = [&](int i) {
    const int j0 = tile_j0(i);
    stage.load(prm, page_of(j0), page_of(j0 + 16), j0, L, kvh, lane, wave);
  };
  if (ntiles > 0) {
    issue(0);
    stage.store(set_of(0), lane, wave);
    if (ntiles > 1) issue(1);
  }
  __syncthreads();
  for (int i = 0; i < ntiles; ++i) {
    compute(tile_j0(i), set_of(i));
    if (i + 1 < ntiles) {
      stage.store(set_of(i + 1), lane, wave);
      if (i + 2 < ntiles) issue(i + 2);
    }
    __syncthreads();
  }

  lsum = wave_sum_pair(lsum);
  lrnd = wave_sum_pair(lrnd);
  const bool any = lsum > 0.0f;
  const float lse_s = any ? (m2 + __log2f(lsum)) * kLn2 : -INFINITY;
  const float inv = any ? 1.0f / lrnd : 0.0f;
  if (col_ok) {
    const size_t slot = ((size_t)bk * prm.nsplit + split) * prm.ncols + col;
    float *po = prm.part_o + slot * D + 4 * hh;
#pragma unroll
    for (int db = 0; db < st::kDB; ++db) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 wv;
#pragma unroll
        for (int j = 0; j < 4; ++j) wv[j] = oacc[db][4 * i + j] * inv;
        *(f32x4 *)(po + 32 * db + 8 * i) = wv;
      }
    }
    if (hh == 0) prm.part_lse[slot] = lse_s;
  }
}

// Merges the splits of one (sequence, KV head, column): W waves, wave w
// taking the splits w, w + W, ...; the threads first reduce the splits' lse
// maximum, then each lane of a wave accumulates D / 64 values of O over its
// wave's splits, and wave 0 adds the W partial sums.  Only splits of a
// sequence that holds keys matter; the others have lse = -inf.  W = 4 when
// there are many splits (the walk over them is the merge's latency), else 1.
template <int D, int kMergeWaves>
__global__ __launch_bounds__(64 * kMergeWaves) void attn_decode_merge_kernel(DecParams prm) {
  constexpr int kPer = D / 64;  // d values per lane
  __shared__ float red[kMergeWaves];
  __shared__ float part_acc[kMergeWaves][64 * kPer];
  __shared__ float part_tot[kMergeWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int col = blockIdx.x % prm.ncols;
  const int bk = blockIdx.x / prm.ncols;
  const int b = bk / prm.Hkv, kvh = bk % prm.Hkv;
  const size_t slot0 = (size_t)bk * prm.nsplit * prm.ncols + col;
  float m = -INFINITY;
  for (int s = tid; s < prm.nsplit; s += 64 * kMergeWaves)
    m = fmaxf(m, prm.part_lse[slot0 + (size_t)s * prm.ncols]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if constexpr (kMergeWaves > 1) {
    if (lane == 0) red[wv] = m;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w) m = fmaxf(m, red[w]);
  }
  // every split wrote its slot (an empty one o = 0, lse = -inf, whose weight
  // exp(-inf - m) is 0), so the walk is branch-free; eight splits per step
  // keep eight loads in flight per lane
  float acc[kPer] = {};
  float tot = 0.0f;
  if (m > -INFINITY) {
    constexpr int kU = 8;
    for (int s0 = wv; s0 < prm.nsplit; s0 += kU * kMergeWaves) {
      float ls[kU], ov[kU][kPer];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int sp = s0 + u * kMergeWaves;
        const bool in = sp < prm.nsplit;
        const size_t slot = slot0 + (size_t)(in ? sp : 0) * prm.ncols;
        ls[u] = in ? prm.part_lse[slot] : -INFINITY;
        const float *po = prm.part_o + slot * D + lane * kPer;
#pragma unroll
        for (int j = 0; j < kPer; ++j) ov[u][j] = po[j];
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const float w = __expf(ls[u] - m);
        tot += w;
#pragma unroll
        for (int j = 0; j < kPer; ++j) acc[j] += w * ov[u][j];
      }
    }
  }
  if constexpr (kMergeWaves > 1) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) part_acc[wv][lane * kPer + j] = acc[j];
    if (lane == 0) part_tot[wv] = tot;
    __syncthreads();
    if (wv != 0) return;
#pragma unroll
    for (int w = 1; w < kMergeWaves; ++w) {
#pragma unroll
      for (int j = 0; j < kPer; ++j) acc[j] += part_acc[w][lane * kPer + j];
      tot += part_tot[w];
    }
  }
  const int g = col / prm.T, t = col % prm.T;
  const size_t row = (size_t)(b * prm.Hq + kvh * prm.G + g) * prm.T + t;
  const float inv = tot > 0.0f ? 1.0f / tot : 0.0f;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const __bf16 x = (__bf16)(acc[j] * inv);
    prm.o[row * D + lane * kPer + j] = __builtin_bit_cast(uint16_t, x);
  }
  if (lane == 0) prm.lse[row] = tot > 0.0f ? m + __logf(tot) : -INFINITY;
}

template <int D>
hipError_t launch_decode_d(const DecodeProblem &p, const DecodePlan &plan, hipStream_t stream) {
  DecParams prm;
  prm.q = static_cast<const uint16_t *>(p.q);
  prm.kc = static_cast<const uint16_t *>(p.k_cache);
  prm.vc = static_cast<const uint16_t *>(p.v_cache);
  prm.table = p.block_table;
  prm.lens = p.seq_lens;
  prm.o = static_cast<uint16_t *>(p.o);
  prm.lse = p.lse;
  prm.part_o = static_cast<float *>(p.workspace);
  prm.part_lse = prm.part_o + plan.part_o_floats;
  prm.B = p.B; prm.Hq = p.Hq; prm.Hkv = p.Hkv; prm.G = p.Hq / p.Hkv; prm.T = p.T;
  prm.ncols = prm.G * p.T;
  prm.ncb = (prm.ncols + 31) / 32;
  prm.ps = p.page_size;
  prm.ps_shift = __builtin_ctz((unsigned)p.page_size);
  prm.num_pages = p.num_pages;
  prm.max_pages = p.max_pages;
  prm.nsplit = plan.nsplit;
  prm.chunk = plan.chunk;
  prm.unit = p.page_size > kKeys ? p.page_size : kKeys;
  const float c = std::fabs(p.scale) * kLog2e;
  prm.c = c < FLT_MIN ? FLT_MIN : c;
  prm.neg = p.scale < 0.0f ? 1 : 0;
  prm.window = p.window;
  const long long groups = (long long)p.B * p.Hkv;
  const long long items = groups * plan.nsplit;
  // more than one column block: W waves per workgroup, one per block, and
  // ceil(ncb / W) workgroups per item
  const int W = prm.ncb >= 4 ? 4 : prm.ncb >= 2 ? 2 : 1;
  const int ngr = (prm.ncb + W - 1) / W;
  const long long wgs = ngr == 1 ? items : (items + 7) / 8 * 8 * ngr;
  if (wgs > 0x7fffffffLL) return hipErrorInvalidValue;
  prm.nwork = (int)items;
  void *args[] = {&prm};
  // K/V bytes the call may read (every split full): a working set that fits
  // the 256 MB last-level cache can stay there from one call to the next
  // and is read with ordinary loads; a larger one is streamed with
  // nontemporal loads (measured: 7-10 % faster at 1.9 GB, 9 % slower at
  // 135 MB, where ordinary loads hit the last-level cache).  Workgroups of
  // one item after the first read its K/V tiles from L2, which a
  // nontemporal load would not have kept: those calls use ordinary loads.
  const double kv_bytes = (double)groups * plan.nsplit * plan.chunk * D * 4.0;
  const bool nt = kv_bytes > kLastLevelCacheBytes && ngr == 1;
  const void *split;
  if (W == 4)
    split = nt ? reinterpret_cast<const void *>(&attn_decode_split_mc_kernel<D, 2, 4>)
               : reinterpret_cast<const void *>(&attn_decode_split_mc_kernel<D, 0, 4>);
  else if (W == 2)
    split = nt ? reinterpret_cast<const void *>(&attn_decode_split_mc_kernel<D, 2, 2>)
               : reinterpret_cast<const void *>(&attn_decode_split_mc_kernel<D, 0, 2>);
  else
    split = nt ? reinterpret_cast<const void *>(&attn_decode_split_kernel<D, 2>)
               : reinterpret_cast<const void *>(&attn_decode_split_kernel<D, 0>);
  hipError_t e = hipLaunchKernel(split, dim3((unsigned)wgs), dim3(64 * W), args, 0, stream);
  if (e != hipSuccess) return e;
  const long long merges = groups * prm.ncols;
  if (merges > 0x7fffffffLL) return hipErrorInvalidValue;
  if (plan.nsplit >= 64)
    return hipLaunchKernel(reinterpret_cast<const void *>(&attn_decode_merge_kernel<D, 4>),
                           dim3((unsigned)merges), dim3(256), args, 0, stream);
  return hipLaunchKernel(reinterpret_cast<const void *>(&attn_decode_merge_kernel<D, 1>),
                         dim3((unsigned)merges), dim3(64), args, 0, stream);
}

}  // namespace

DecodePlan plan_decode(int B, int Hq, int Hkv, int T, int d, int page_size, int max_seq_len,
                       int window) {
  DecodePlan plan{};
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || T <= 0 || page_size <= 0 || max_seq_len <= 0) return plan;
  const int unit = page_size > kKeys ? page_size : kKeys;
  // keys a sequence's queries can see: all of them, or the last window + T - 1
  // (plus up to one unit of rounding at the start)
  long long span = max_seq_len;
  if (window > 0 && (long long)window + T - 1 + unit < span) span = (long long)window + T - 1 + unit;
  const long long max_chunk = (long long)kMaxEntries * page_size;  // one table entry per lane
  // about 4096 single-wave workgroups when every sequence is max_seq_len
  // long: four times the 1024 the GPU holds at once at d = 128 (254 VGPRs
  // and 144 AGPRs: one wave per SIMD).  Shorter sequences leave their last
  // splits empty, so a typical call runs in a few rounds of workgroups.
  // (Measured on 8 sequences of 12k..102k keys: 3072-4096 in total is 3 %
  // faster than 8192 and 13 % faster than 2048.)
  // With more than 32 columns each key range is one workgroup per 32-column
  // block, so the count is of (range, block) pairs.
  const long long ncb = ((long long)(Hq / Hkv) * T + 31) / 32;
  const long long groups = (long long)B * Hkv;
  long long want = (4096 + groups * ncb - 1) / (groups * ncb);
  long long chunk = (span + want - 1) / want;
  // with several column blocks a workgroup of several waves takes each
  // split: at least 1024 keys (32 tiles) per split (measured: 64 heads on
  // one KV head +17 % against 512 keys; 16 heads x 4 tokens, already at
  // 1024, lose 16 % at 2048)
  if (ncb > 1 && chunk < 1024) chunk = 1024;
  chunk = (chunk + unit - 1) / unit * unit;
  if (chunk < unit) chunk = unit;
  if (chunk > max_chunk) chunk = max_chunk;
  plan.chunk = (int)chunk;
  plan.nsplit = (int)((span + chunk - 1) / chunk);
  const long long ncols = (long long)(Hq / Hkv) * T;
  plan.part_o_floats = (size_t)groups * plan.nsplit * ncols * d;
  plan.part_lse_floats = (size_t)groups * plan.nsplit * ncols;
  return plan;
}

hipError_t launch_decode(const DecodeProblem &p, const DecodePlan &plan, hipStream_t stream) {
  return p.d == 128 ? launch_decode_d<128>(p, plan, stream) : launch_decode_d<64>(p, plan, stream);
}

// Scratch of the allocation-free decode entry point: the split partials
// (partial O then partial lse, as in the workspace of attn_decode_paged).
// Every split writes its slot before the merge reads it, so nothing needs
// clearing between calls.  One copy per GPU, at its own address.
static __device__ __align__(256) float scratch[ATTN_DECODE_NOALLOC_MAX_BYTES / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t decode_noalloc_scratch(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace attn
