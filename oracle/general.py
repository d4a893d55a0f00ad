"""NumPy float64 oracle for structured masks on packed variable-length batches.

TEST INFRASTRUCTURE ONLY: see the package docstring for who may import this.

Two structures from the pages, both exact attention with a mask:

* Block-diagonal packing: "Efficient attention: long context and
  sub-quadratic variants", section "Against the real libraries", names
  xformers' BlockDiagonalMask among the structured masks that reach a kernel
  as iteration bounds.  Sequences of different lengths are packed one after
  another; a token attends only within its own sequence, i.e. the plain
  definition applied to each sequence separately.  Sequence b is rows
  cu[b] .. cu[b+1]-1 of every head's [total_rows][d] slice.
* Local plus global attention (Longformer): same page, section
  "Sliding-window and local attention", and "Efficient Attention:
  FlashAttention, Sparse, Linear", section 45.2.2: each token attends to a
  fixed neighbourhood (the diagonal band), and a few designated global
  tokens attend to everything and are attended to by everything.

Within one sequence of N rows, row i sees key j iff

    (not causal or j <= i) and
    (i < n_global or j < n_global or
     ((window <= 0 or j > i - window) and (radius <= 0 or |i - j| <= radius)))

The global tokens are the first n_global positions of each sequence (reading
15: the classification and question tokens lead a Longformer input);
``radius`` is the half-width of the band (Longformer's window of 512 is
radius 256); ``window`` is the causal sliding window of the forward.  With
n_global = 0 and radius = 0 the rule is the forward's.  Every row sees at
least itself, so no row is empty.

Masked scores are -inf before the softmax ("Implementation, twice"); lse is
the natural-log logsumexp of the scaled scores over the visible set.  Each
row block is computed against the explicit set of keys its rows may see
(the global keys plus the band), gathered by index; keys outside the set
would get weight exactly 0.
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .attention import as_f64


def visible(i, j, causal=False, window=0, radius=0, n_global=0):
    """The rule above for one (row, key) pair of one sequence (Python ints)."""
    if causal and j > i:
        return False
    if i < n_global or j < n_global:
        return True
    if window > 0 and not j > i - window:
        return False
    if radius > 0 and abs(i - j) > radius:
        return False
    return True


def visible_block(i, j, causal=False, window=0, radius=0, n_global=0):
    """The same rule over broadcast integer arrays of rows i and keys j."""
    vis = np.ones(np.broadcast(i, j).shape, dtype=bool)
    if causal:
        vis &= j <= i
    local = np.ones_like(vis)
    if window > 0:
        local &= j > i - window
    if radius > 0:
        local &= np.abs(i - j) <= radius
    return vis & ((i < n_global) | (j < n_global) | local)


def _candidate_keys(r0, r1, N, causal, window, radius, n_global):
    """Sorted key indices any row of [r0, r1) may see (a superset)."""
    if r0 < n_global:
        return np.arange(r1 if causal else N)
    hi = r1 if causal else N
    lo = 0
    if window > 0:
        lo = max(lo, r0 - window + 1)
    if radius > 0:
        lo = max(lo, r0 - radius)
        hi = min(hi, r1 + radius)
    band = np.arange(lo, hi)
    glob = np.arange(min(n_global, hi))
    return np.union1d(glob, band)


def attention_general(q, k, v, scale, cu_seqlens, causal=False, window=0, radius=0,
                      n_global=0, block=128, workers=1):
    """Exact attention over packed sequences with the rule above.

    q: (Hq, total, d); k, v: (Hkv, total, d); cu_seqlens: B + 1 offsets.
    Returns o (Hq, total, d) and lse (Hq, total), float64.
    """
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    Hq, total, d = q.shape
    Hkv = k.shape[0]
    if k.shape != (Hkv, total, d) or v.shape != k.shape or Hq % Hkv:
        raise ValueError("q (Hq, total, d), k and v (Hkv, total, d), Hq % Hkv == 0")
    if window > 0 and not causal:
        raise ValueError("window > 0 requires causal")
    cu = [int(x) for x in cu_seqlens]
    if cu[0] != 0 or cu[-1] != total or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must rise from 0 to total")
    sigma = float(np.float32(scale))
    if not math.isfinite(sigma):
        raise ValueError("scale must be finite")
    G = Hq // Hkv
    o = np.zeros((Hq, total, d), dtype=np.float64)
    lse = np.zeros((Hq, total), dtype=np.float64)

    def one(task):
        h, b = task
        s0, N = cu[b], cu[b + 1] - cu[b]
        if N == 0:
            return
        qh = as_f64(q[h, s0:s0 + N])
        kh = as_f64(k[h // G, s0:s0 + N])
        vh = as_f64(v[h // G, s0:s0 + N])
        for r0 in range(0, N, block):
            r1 = min(N, r0 + block)
            keys = _candidate_keys(r0, r1, N, causal, window, radius, n_global)
            vis = visible_block(np.arange(r0, r1)[:, None], keys[None, :], causal, window,
                                radius, n_global)
            s = sigma * (qh[r0:r1] @ kh[keys].T)
            s = np.where(vis, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            den = e.sum(axis=1, keepdims=True)
            o[h, s0 + r0:s0 + r1] = (e / den) @ vh[keys]
            lse[h, s0 + r0:s0 + r1] = (m + np.log(den))[:, 0]

    tasks = [(h, b) for h in range(Hq) for b in range(len(cu) - 1)]
    if workers <= 1:
        for t in tasks:
            one(t)
    else:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(one, tasks))
    return o, lse
