"""The attention-forward workloads and their algorithmic counts.

Shapes come from the pages:

* 128k context, 32 heads, d = 128 -- "Efficient attention: long context and
  sub-quadratic variants", section "The quadratic wall, stated concretely".
* window w = 4096 at N = 131072 -- same page, "Sliding-window and local
  attention".
* (2, 32, 8192, 128) causal -- "Efficient Attention: Flash Attention,
  Sliding Window, Sparse", section "Code".
* 64 query heads over 8 KV heads -- "Attention Mechanism Variants Beyond
  Self-Attention", section "Multi-Query and Grouped-Query Attention".

Counting convention: one unmasked score costs 4*d FLOPs (2*d for q.k and 2*d
for its share of P V), which is the "2N^2 d ... the same again" count of
"The quadratic wall, stated concretely"; masked or computed-but-discarded
tile entries never count.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

MI355X_BF16_DENSE_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 bf16 FLOP/CU/clk
MI355X_HBM_GBPS = 8000.0
MI355X_FP8_DENSE_TFLOPS = 5033.2  # twice the bf16 rate


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    causal: bool
    window: int
    seed: int
    q_mult: float = 1.0
    scale: float = field(default=0.0)
    sampled_rows: int = 0  # 0: the oracle covers every row

    @property
    def sm_scale(self) -> float:
        return self.scale if self.scale else 1.0 / math.sqrt(self.d)


def visible_scores_per_head(N: int, causal: bool, window: int) -> int:
    """Number of (i, j) pairs with j visible from i, for one head."""
    if not causal:
        return N * N
    if window <= 0 or window >= N:
        return N * (N + 1) // 2
    # rows i < w see i + 1 keys, rows i >= w see exactly w keys
    return window * (window + 1) // 2 + (N - window) * window


def visible_scores(w: Workload) -> int:
    return w.B * w.Hq * visible_scores_per_head(w.N, w.causal, w.window)


def flops(w: Workload) -> int:
    return 4 * w.d * visible_scores(w)


def bwd_flops(w: Workload) -> int:
    """Backward: five 2*d contractions per unmasked score (recomputed S = QK^T,
    dP = dO V^T, dV += P^T dO, dQ += dS K, dK += dS^T Q)."""
    return 10 * w.d * visible_scores(w)


def algorithmic_bytes(w: Workload) -> int:
    """Q, K, V read once, O (bf16) and lse (fp32) written once."""
    return 2 * w.B * w.N * w.d * (2 * w.Hq + 2 * w.Hkv) + 4 * w.B * w.Hq * w.N


WORKLOADS = {
    "c1_noncausal_mha": Workload("c1_noncausal_mha", 1, 2, 2, 256, 64, False, 0, 1,
                                 scale=1.0 / 8.0),
    "c2_causal_mha": Workload("c2_causal_mha", 2, 32, 32, 8192, 128, True, 0, 2),
    "c2_causal_mha_sharp": Workload("c2_causal_mha_sharp", 2, 32, 32, 8192, 128, True, 0,
                                    2, q_mult=4.0),
    "c3_causal_window": Workload("c3_causal_window", 1, 32, 32, 32768, 128, True, 4096, 3),
    "c4_causal_gqa": Workload("c4_causal_gqa", 1, 64, 8, 16384, 128, True, 0, 4),
    "c5_long_causal": Workload("c5_long_causal", 1, 32, 32, 131072, 128, True, 0, 5,
                               sampled_rows=256),
    "c5_long_window": Workload("c5_long_window", 1, 32, 32, 131072, 128, True, 4096, 5,
                               sampled_rows=256),
}


# ---------------------------------------------------------------------------
# Paged decode workloads: the serving-side sibling ("FlashAttention: exact
# attention, IO-aware", PagedAttention).  Shapes from the same pages: the
# 64 / 8 GQA heads and d = 128, contexts up to the 128k of "The quadratic
# wall, stated concretely", the window 4096 of "Sliding-window and local
# attention"; a batch of sequences with a seeded uniform length mix.
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    Hq: int
    Hkv: int
    T: int
    d: int
    page_size: int
    max_len: int
    seed: int
    window: int = 0

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


def decode_visible_keys(w: DecodeWorkload, L: int) -> int:
    """Cached tokens any query of a length-L sequence sees (each is read once)."""
    if w.window > 0:
        return min(L, w.window + w.T - 1)
    return L


def decode_bytes(w: DecodeWorkload, lens) -> int:
    """Algorithmic HBM bytes of one call: the visible K and V rows once, q and o
    (bf16), lse (fp32), the page-table entries and lengths read."""
    kv = sum(decode_visible_keys(w, L) for L in lens) * w.Hkv * w.d * 2 * 2
    qo = 2 * w.B * w.Hq * w.T * w.d * 2 + 4 * w.B * w.Hq * w.T
    table = sum((L + w.page_size - 1) // w.page_size for L in lens) * 4 + 4 * w.B
    return kv + qo + table


DECODE_WORKLOADS = {
    "d1_decode_gqa_128k": DecodeWorkload("d1_decode_gqa_128k", 8, 64, 8, 1, 128, 64, 131072, 21),
    "d2_decode_mha_8k": DecodeWorkload("d2_decode_mha_8k", 32, 32, 32, 1, 128, 16, 8192, 22),
    "d3_decode_window_spec4": DecodeWorkload("d3_decode_window_spec4", 8, 64, 8, 4, 128, 256,
                                             131072, 23, window=4096),
    # multi-query: one KV head for 64 query heads (64 columns per KV head)
    "d4_decode_mqa_128k": DecodeWorkload("d4_decode_mqa_128k", 8, 64, 1, 1, 128, 64, 131072, 24),
    # 16 query heads per KV head x 4 new tokens (64 columns per KV head)
    "d5_decode_gqa16_spec4": DecodeWorkload("d5_decode_gqa16_spec4", 8, 32, 2, 4, 128, 64,
                                            131072, 25),
}


# ---------------------------------------------------------------------------
# Packed variable-length batches with structured masks (block-diagonal
# packing; Longformer band + global tokens).  Shapes: a packed batch of
# documents with a seeded uniform length mix at the 32 / 8 GQA heads, d = 128;
# Longformer at its 4096-token inputs, band 512 (radius 256), a handful (16)
# of global tokens, 12 heads of d = 64.
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class VarlenWorkload:
    name: str
    lens: tuple
    Hq: int
    Hkv: int
    d: int
    causal: bool
    window: int = 0
    radius: int = 0
    n_global: int = 0
    seed: int = 0

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def total(self) -> int:
        return sum(self.lens)


def visible_pairs_general(N: int, causal: bool, window: int, radius: int, n_global: int) -> int:
    """(row, key) pairs a sequence of N rows sees under the structured-mask
    rule (global rows see every key they may; other rows the global keys
    plus the band), by intervals per row."""
    total = 0
    for i in range(N):
        hi_c = i + 1 if causal else N
        if i < n_global:
            total += hi_c
            continue
        lo, hi = 0, hi_c
        if window > 0:
            lo = max(lo, i - window + 1)
        if radius > 0:
            lo = max(lo, i - radius)
            hi = min(hi, i + radius + 1)
        total += max(0, hi - lo) + max(0, min(n_global, hi_c, lo))
    return total


def varlen_flops(w: VarlenWorkload) -> int:
    return 4 * w.d * w.Hq * sum(visible_pairs_general(L, w.causal, w.window, w.radius,
                                                      w.n_global) for L in w.lens)


def _lens(B: int, max_len: int, seed: int) -> tuple:
    import numpy as np
    rng = np.random.default_rng(seed)
    return tuple(int(x) for x in rng.integers(1, max_len + 1, size=B))


VARLEN_WORKLOADS = {
    "v1_packed_causal_gqa": VarlenWorkload("v1_packed_causal_gqa", _lens(16, 8192, 31), 32, 8,
                                           128, True, seed=31),
    "l1_longformer_4k": VarlenWorkload("l1_longformer_4k", (4096,) * 8, 12, 12, 64, False,
                                       radius=256, n_global=16, seed=32),
}
