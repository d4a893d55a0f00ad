"""NumPy float64 oracle for the gradients of exact attention.

TEST INFRASTRUCTURE ONLY: see the package docstring for who may import this.

"Efficient attention: long context and sub-quadratic variants", section
"Against the real libraries", names a recompute-based backward pass next to
the exact forward; what such a pass returns is the gradient of the forward
definition.  With the forward written out as

    s = sigma * Q K^T (masked to -inf),  P = softmax_rows(s),  O = P V,

and an upstream gradient dO of some loss L with respect to O, the chain rule
gives, per (batch, query head), with K and V those of the head's KV head:

    dV    = P^T dO
    dP    = dO V^T
    Delta = rowsum(dO * O)                  (one value per query row)
    dS    = P * (dP - Delta)                (softmax Jacobian, row by row)
    dQ    = sigma * dS K
    dK    = sigma * dS^T Q

(the masked entries have P = 0 and so dS = 0).  A KV head shared by G query
heads ("Attention Mechanism Variants Beyond Self-Attention", section
"Multi-Query and Grouped-Query Attention": the KV heads are repeated, so
each copy's gradient flows back to the one stored head) receives the sum of
the G heads' dK and dV.

The same row blocking as the forward oracle: each block of query rows is
multiplied against the key span its rows can see; keys outside it have
P = 0 and contribute nothing.
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .attention import as_f64, check_shapes, rows_probabilities, row_blocks


def attention_backward(q, k, v, do, scale, causal=False, window=0, block=256, workers=1):
    """Gradients of sum(O * do) with respect to q, k and v.

    Parameters
    ----------
    q, do : (B, Hq, N, d) arrays, any float dtype (widened to float64 one
        slice at a time).
    k, v : (B, Hkv, N, d) arrays.
    scale, causal, window : as for the forward (the float32 value of scale
        is used, widened).
    block : query rows per block.
    workers : thread-pool size over (batch, query head) pairs.

    Returns ``(dq, dk, dv)`` in float64 with the shapes of q, k and v.
    """
    q, k, v, do = np.asarray(q), np.asarray(k), np.asarray(v), np.asarray(do)
    B, Hq, Hkv, N, d = check_shapes(q, k, v, causal, window)
    if do.shape != q.shape:
        raise ValueError("do must have the shape of q")
    sigma = float(np.float32(scale))
    if not math.isfinite(sigma):
        raise ValueError("scale must be finite")
    G = Hq // Hkv
    dq = np.zeros((B, Hq, N, d), dtype=np.float64)
    dk = np.zeros((B, Hkv, N, d), dtype=np.float64)
    dv = np.zeros((B, Hkv, N, d), dtype=np.float64)
    rows = np.arange(N)
    blocks = row_blocks(rows, N, causal, window, block)

    def one_head(bh):
        # one (batch, query head): writes its own dq slice and returns its
        # contributions to its KV head's dk and dv
        b, h = divmod(bh, Hq)
        kvh = h // G
        kh, vh = as_f64(k[b, kvh]), as_f64(v[b, kvh])
        qh, doh = as_f64(q[b, h]), as_f64(do[b, h])
        dkh = np.zeros((N, d), dtype=np.float64)
        dvh = np.zeros((N, d), dtype=np.float64)
        for r0, r1 in blocks:
            sel = rows[r0:r1]
            p, lo, hi, _ = rows_probabilities(qh, kh, sel, sigma, causal, window, N)
            dos = doh[sel]
            o = p @ vh[lo:hi]
            delta = np.einsum("ij,ij->i", dos, o)
            dvh[lo:hi] += p.T @ dos
            dp = dos @ vh[lo:hi].T
            ds = p * (dp - delta[:, None])
            dq[b, h, sel] = sigma * (ds @ kh[lo:hi])
            dkh[lo:hi] += sigma * (ds.T @ qh[sel])
        return dkh, dvh

    if workers <= 1:
        parts = [one_head(bh) for bh in range(B * Hq)]
    else:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            parts = list(ex.map(one_head, range(B * Hq)))
    # the G query heads of a KV head add up in head order
    for bh, (dkh, dvh) in enumerate(parts):
        b, h = divmod(bh, Hq)
        dk[b, h // G] += dkh
        dv[b, h // G] += dvh
    return dq, dk, dv
