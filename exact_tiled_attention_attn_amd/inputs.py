"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no attention arithmetic: it only draws numbers.  Both the
HIP path and the CPU oracle receive exactly the tensors made here.

Recipe
------
Q, K, V are i.i.d. N(0, 1) draws in float32 from
``torch.Generator().manual_seed(seed)``, taken in the order Q, K, V and,
inside each tensor, one (N, d) slice per (batch, head) in row-major order,
then rounded to bfloat16 with round-to-nearest-even (``Tensor.to``).  The
per-slice drawing keeps host memory bounded at the longest shapes.

The upstream gradient dO of the backward is drawn the same way, from its own
seed, as one (B, Hq, N, d) tensor of N(0, 1) values rounded to bfloat16.
"""

from __future__ import annotations

import numpy as np
import torch


def _draw(gen: torch.Generator, B: int, H: int, N: int, d: int) -> torch.Tensor:
    out = torch.empty((B, H, N, d), dtype=torch.bfloat16)
    for b in range(B):
        for h in range(H):
            out[b, h] = torch.randn((N, d), generator=gen, dtype=torch.float32).to(
                torch.bfloat16)
    return out


def make_qkv(B: int, Hq: int, Hkv: int, N: int, d: int, seed: int):
    """Return bf16 CPU tensors (q, k, v) shaped (B,Hq,N,d), (B,Hkv,N,d) x 2."""
    gen = torch.Generator().manual_seed(int(seed))
    q = _draw(gen, B, Hq, N, d)
    k = _draw(gen, B, Hkv, N, d)
    v = _draw(gen, B, Hkv, N, d)
    return q, k, v


def make_dout(B: int, Hq: int, N: int, d: int, seed: int) -> torch.Tensor:
    """Return a bf16 CPU tensor dO shaped (B, Hq, N, d)."""
    gen = torch.Generator().manual_seed(int(seed))
    return _draw(gen, B, Hq, N, d)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Widen a bf16/fp32 CPU tensor to a float64 NumPy array (exact)."""
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def sample_rows(N: int, count: int, seed: int, edges=(0, 1, 127, 128, 4095, 4096)) -> np.ndarray:
    """Sorted distinct query rows: `count` uniform draws plus edge rows.

    Drawn with ``numpy.random.default_rng(seed)`` without replacement; the
    edge rows (and N - 1) are added when they exist.
    """
    rng = np.random.default_rng(int(seed))
    picks = rng.choice(N, size=min(count, N), replace=False)
    extra = [e for e in edges if e < N] + [N - 1]
    return np.unique(np.concatenate([picks, np.asarray(extra, dtype=np.int64)]))
