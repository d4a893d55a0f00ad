"""NumPy float64 oracle for decode attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY: see the package docstring for who may import this.

"Efficient attention: long context and sub-quadratic variants", section
"FlashAttention: exact attention, IO-aware", describes the serving-side
PagedAttention: the KV cache lives in fixed-size pages with a per-sequence
page table, attention gathers K and V through that table, sequences may
share pages, and nothing is approximated.  So the result is plain exact
attention over the gathered cache:

* sequence b holds L_b = seq_lens[b] cached tokens; token j of it is slot
  j % page_size of physical page block_table[b][j // page_size];
* its T newest tokens are the queries: query t sits at position
  L_b - T + t and sees the cached keys j <= that position (the causal rule
  of "Implementation, twice"), and with a window w > 0 only j > pos - w
  ("Sliding-window and local attention");
* query head h reads KV head h // (Hq / Hkv) ("Attention Mechanism Variants
  Beyond Self-Attention", "Multi-Query and Grouped-Query Attention");
* scores sigma * q . k (sigma = float32(scale) widened), softmax over the
  visible keys, output sum_j p_j v_j and lse = ln sum_j exp(s_j) (natural
  log of the scaled scores, as for the forward).

A query that sees no key (L_b - T + t < 0, only possible when the caller
passes fewer cached tokens than queries) gets o = 0 and lse = -inf.

The gather is written out with NumPy fancy indexing, the attention per
query as the plain definition over its visible keys.  ``merge_partials``
states the rule that combines results over disjoint key sets (a split-KV
schedule computes one part per key range).
"""

from __future__ import annotations

import math

import numpy as np

from .attention import as_f64


def gather_pages(cache, table_row, length):
    """The first ``length`` tokens of one sequence from a paged cache.

    cache: (num_pages, page_size, Hkv, d); table_row: 1-D page indices.
    Returns (length, Hkv, d): token j is cache[table_row[j // ps], j % ps].
    """
    ps = cache.shape[1]
    j = np.arange(length)
    pages = np.asarray(table_row)[j // ps]
    return cache[pages, j % ps]


def decode_paged(q, k_cache, v_cache, block_table, seq_lens, scale, window=0):
    """Exact attention of the T newest tokens of each sequence over its cache.

    q: (B, Hq, T, d); k_cache, v_cache: (num_pages, page_size, Hkv, d);
    block_table: (B, max_pages) integers; seq_lens: (B,) integers.
    Returns (o, lse): (B, Hq, T, d) and (B, Hq, T) float64.
    """
    q = np.asarray(q)
    B, Hq, T, d = q.shape
    num_pages, ps, Hkv, dk = k_cache.shape
    if v_cache.shape != k_cache.shape or dk != d:
        raise ValueError("k_cache and v_cache must be (num_pages, page_size, Hkv, d)")
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    block_table = np.asarray(block_table)
    seq_lens = np.asarray(seq_lens)
    G = Hq // Hkv
    sigma = float(np.float32(scale))
    if not math.isfinite(sigma):
        raise ValueError("scale must be finite")
    o = np.zeros((B, Hq, T, d), dtype=np.float64)
    lse = np.full((B, Hq, T), -np.inf, dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        if (L + ps - 1) // ps > block_table.shape[1]:
            raise ValueError("seq_lens[b] exceeds the page table row")
        kb = as_f64(gather_pages(k_cache, block_table[b], L))  # (L, Hkv, d)
        vb = as_f64(gather_pages(v_cache, block_table[b], L))
        for h in range(Hq):
            kvh = h // G
            qh = as_f64(q[b, h])
            for t in range(T):
                pos = L - T + t
                if pos < 0:
                    continue
                lo = max(0, pos - window + 1) if window > 0 else 0
                s = sigma * (kb[lo:pos + 1, kvh] @ qh[t])
                m = s.max()
                e = np.exp(s - m)
                den = e.sum()
                o[b, h, t] = (e / den) @ vb[lo:pos + 1, kvh]
                lse[b, h, t] = m + math.log(den)
    return o, lse


def merge_partials(o_parts, lse_parts):
    """Combine attention results over disjoint key sets.

    o_parts: (S, ..., d) outputs normalised over their own key sets;
    lse_parts: (S, ...) their natural-log logsumexps (-inf for an empty
    set).  Returns the (o, lse) of the union: lse = ln sum_s exp(lse_s),
    o = sum_s exp(lse_s - lse) o_s -- the rescaling by exp(m_old - m_new)
    of the running softmax in "FlashAttention: exact attention, IO-aware",
    applied once per part.
    """
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    o_parts = np.asarray(o_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    safe = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(lse_parts - safe)
    tot = w.sum(axis=0)
    with np.errstate(divide="ignore"):
        lse = np.where(tot > 0, safe + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    o = (w[..., None] * o_parts).sum(axis=0) / np.where(tot > 0, tot, 1.0)[..., None]
    return o, lse
