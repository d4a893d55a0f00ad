"""Pure-Python brute force for exact attention -- TEST INFRASTRUCTURE ONLY.

Every (query, key) pair is visited with plain loops, the visibility test is
evaluated per pair, and every sum is an exactly rounded ``math.fsum``.
No blocking, no NumPy.  It exists to pin the NumPy oracle on tiny shapes.

Definition followed ("Efficient attention: long context and sub-quadratic
variants", sections "Sliding-window and local attention" and
"Implementation, twice"; GQA head map from "Attention Mechanism Variants
Beyond Self-Attention", section "Multi-Query and Grouped-Query Attention"):
row i sees key j iff (not causal or j <= i) and (window <= 0 or j > i - w);
weights are the softmax of sigma * q_i . k_j over that set; other keys get
weight 0; query head h reads KV head h // (Hq // Hkv).
"""

from __future__ import annotations

import math
import struct


def _f32(x: float) -> float:
    """Round a Python float to the nearest float32 and widen it back."""
    return struct.unpack("f", struct.pack("f", x))[0]


def brute_attention(q, k, v, scale, causal=False, window=0):
    """q: nested lists [B][Hq][N][d]; k, v: [B][Hkv][N][d] (Python floats).

    Returns (o, lse) as nested lists [B][Hq][N][d] and [B][Hq][N].
    """
    B, Hq, N, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv = len(k[0])
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    sigma = _f32(float(scale))
    o = [[[[0.0] * d for _ in range(N)] for _ in range(Hq)] for _ in range(B)]
    lse = [[[0.0] * N for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            kvh = h // G
            for i in range(N):
                seen = []
                for j in range(N):
                    ok = True
                    if causal and j > i:
                        ok = False
                    if window > 0 and not j > i - window:
                        ok = False
                    if ok:
                        seen.append(j)
                if not seen:
                    raise AssertionError("row with no visible key")
                score = {}
                for j in seen:
                    score[j] = sigma * math.fsum(
                        q[b][h][i][t] * k[b][kvh][j][t] for t in range(d))
                top = max(score.values())
                w = {j: math.exp(score[j] - top) for j in seen}
                total = math.fsum(w.values())
                lse[b][h][i] = top + math.log(total)
                for t in range(d):
                    o[b][h][i][t] = math.fsum(w[j] * v[b][kvh][j][t] for j in seen) / total
    return o, lse
