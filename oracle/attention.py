"""NumPy float64 oracle for exact (optionally masked, optionally GQA) attention.

TEST INFRASTRUCTURE ONLY: see the package docstring for who may import this.

The computation is the plain definition, written out:

    s_ij   = sigma * <q_i, k_j>                         (float64)
    V_i    = { j : (not causal or j <= i) and (window <= 0 or j > i - window) }
    m_i    = max_{j in V_i} s_ij
    l_i    = sum_{j in V_i} exp(s_ij - m_i)
    lse_i  = m_i + ln(l_i)
    p_ij   = exp(s_ij - m_i) / l_i   for j in V_i, exactly 0 otherwise
    o_i    = sum_j p_ij v_j

Sources (page title, section):

* "Efficient attention: long context and sub-quadratic variants",
  "Implementation, twice": the core function divides q k^T by sqrt(d),
  fills masked scores with -inf *before* the softmax (masked weights are
  exactly zero and each row renormalises over what it sees), and the window
  mask is ``(j <= i) & (j > i - window)`` -- at most ``window`` keys per row.
  Same page, "Sliding-window and local attention": row i sees i - w < j <= i
  in the causal case.
* Same page, "Using it on a real shape of problem": a window >= T is exactly
  full causal attention.
* "Attention Mechanism Variants Beyond Self-Attention", "Multi-Query and
  Grouped-Query Attention": ``kv_repeat = num_heads // num_kv_heads`` and
  ``repeat_interleave(kv_repeat, dim=1)``, i.e. query head h uses KV head
  h // kv_repeat.

sigma is the float32 value of ``scale`` widened to float64, because that is
the value a caller passes through the C interface.

The only restructuring is a row blocking: each block of query rows is
multiplied against the contiguous key span that any of its rows can see,
and the exact element mask is applied inside the span.  Keys outside the
span would receive weight exactly 0, so this is the same definition, not an
approximation.  A thread pool over (batch, head) slices is optional and does
not change any value.
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np


def check_shapes(q, k, v, causal, window):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be (B, H, N, d)")
    B, Hq, N, d = q.shape
    if k.shape[0] != B or k.shape[2] != N or k.shape[3] != d or v.shape != k.shape:
        raise ValueError("k and v must be (B, Hkv, N, d) matching q")
    Hkv = k.shape[1]
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    if window > 0 and not causal:
        # The window is defined only for the causal case ("Sliding-window and
        # local attention"); the oracle refuses the undefined combination.
        raise ValueError("window > 0 requires causal")
    return B, Hq, Hkv, N, d


def visible_span(i: int, N: int, causal: bool, window: int) -> tuple[int, int]:
    """Half-open key range [lo, hi) that row i can see.

    Row i sees j <= i when causal and j > i - window when window > 0
    ("Sliding-window and local attention").  The window clamps at key 0, so
    any window >= i + 1 behaves like plain causal for that row.
    """
    hi = i + 1 if causal else N
    lo = max(0, i - window + 1) if window > 0 else 0
    return lo, hi


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """KV head read by query head h: ``repeat_interleave`` puts copy h of the
    repeated KV heads at index h // (Hq // Hkv) ("Multi-Query and
    Grouped-Query Attention")."""
    return h // (Hq // Hkv)


def _visible_mask(rows: np.ndarray, lo: int, hi: int, causal: bool, window: int):
    """Boolean (len(rows), hi - lo): True where key j may be seen by row i."""
    i = rows[:, None]
    j = np.arange(lo, hi)[None, :]
    allowed = np.ones((rows.shape[0], hi - lo), dtype=bool)
    if causal:
        allowed &= j <= i
    if window > 0:
        allowed &= j > i - window
    return allowed


def rows_probabilities(qh, kh, rows, sigma, causal, window, N):
    """Softmax weights of the given query rows of one (batch, head).

    Returns ``(p, lo, hi, lse)``: p is (len(rows), hi - lo) float64 over the
    union key span [lo, hi) of the rows, exactly 0 where a key is masked.
    """
    spans = [visible_span(int(i), N, causal, window) for i in rows]
    lo = min(s[0] for s in spans)
    hi = max(s[1] for s in spans)
    s = sigma * (qh[rows] @ kh[lo:hi].T)  # float64 scores
    allowed = _visible_mask(rows, lo, hi, causal, window)
    if not allowed.any(axis=1).all():
        raise AssertionError("a query row has no visible key")
    s = np.where(allowed, s, -np.inf)  # -inf before the softmax
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)  # masked entries: exp(-inf) == 0 exactly
    l = e.sum(axis=1)
    lse = m[:, 0] + np.log(l)
    p = e / l[:, None]
    return p, lo, hi, lse


def _rows_block(qh, kh, vh, rows, sigma, causal, window, N):
    """Exact attention for the given query rows of one (batch, head)."""
    p, lo, hi, lse = rows_probabilities(qh, kh, rows, sigma, causal, window, N)
    o = p @ vh[lo:hi]
    return o, lse


def row_blocks(rows, N, causal, window, block):
    """Cut ``rows`` into runs of at most ``block`` entries whose union key span
    stays within twice the widest single-row span (so scattered rows under a
    window are not multiplied against keys none of them can see)."""
    if rows.size == 0:
        return []
    widest = max(visible_span(int(i), N, causal, window)[1]
                 - visible_span(int(i), N, causal, window)[0] for i in (rows.min(), rows.max()))
    if window > 0:
        widest = max(widest, min(window, N))
    limit = 2 * max(widest, block)
    out, start = [], 0
    lo, hi = visible_span(int(rows[0]), N, causal, window)
    for n in range(1, rows.size + 1):
        if n == rows.size:
            out.append((start, n))
            break
        l2, h2 = visible_span(int(rows[n]), N, causal, window)
        nlo, nhi = min(lo, l2), max(hi, h2)
        if n - start >= block or nhi - nlo > limit:
            out.append((start, n))
            start, lo, hi = n, l2, h2
        else:
            lo, hi = nlo, nhi
    return out


def as_f64(x):
    x = np.asarray(x)
    if x.dtype != np.float64:
        x = x.astype(np.float64)
    return x


def attention_rows(q, k, v, scale, causal=False, window=0, rows=None, block=256,
                   workers=1):
    """Exact attention for a subset of query rows (the same rows in every head).

    Parameters
    ----------
    q : (B, Hq, N, d) array, any float dtype; each (batch, head) slice is
        widened to float64 (exact for bf16/fp32 values) when it is used.
    k, v : (B, Hkv, N, d) arrays.
    scale : softmax scale; the float32 value is used, widened.
    causal, window : mask flags (window <= 0 means no window).
    rows : 1-D integer array of query positions, or None for all rows.
    block : rows per block.
    workers : thread-pool size over (batch, head) slices.

    Returns ``(o, lse)`` with shapes (B, Hq, R, d) and (B, Hq, R) in float64,
    R = len(rows).
    """
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    B, Hq, Hkv, N, d = check_shapes(q, k, v, causal, window)
    sigma = float(np.float32(scale))
    if not math.isfinite(sigma):
        raise ValueError("scale must be finite")
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= N):
        raise ValueError("rows out of range")
    R = rows.shape[0]
    o = np.empty((B, Hq, R, d), dtype=np.float64)
    lse = np.empty((B, Hq, R), dtype=np.float64)

    blocks = row_blocks(rows, N, causal, window, block)

    def one_slice(bh):
        b, h = divmod(bh, Hq)
        kvh = kv_head_of(h, Hq, Hkv)
        # widened one slice at a time so long inputs stay float32 in memory
        qh, kh, vh = as_f64(q[b, h]), as_f64(k[b, kvh]), as_f64(v[b, kvh])
        for r0, r1 in blocks:
            sel = rows[r0:r1]
            ob, lb = _rows_block(qh, kh, vh, sel, sigma, causal, window, N)
            o[b, h, r0:r1] = ob
            lse[b, h, r0:r1] = lb

    if workers <= 1:
        for bh in range(B * Hq):
            one_slice(bh)
    else:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(one_slice, range(B * Hq)))
    return o, lse


def attention_forward(q, k, v, scale, causal=False, window=0, block=256, workers=1):
    """Exact attention over every query row: returns float64 (o, lse)."""
    return attention_rows(q, k, v, scale, causal=causal, window=window, rows=None,
                          block=block, workers=workers)
