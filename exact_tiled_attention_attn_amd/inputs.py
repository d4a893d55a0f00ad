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

Packed variable-length batches (``make_packed_qkv``): Q, K, V of the whole
packed batch drawn like the dense tensors, one (total, d) slice per head;
the lengths of the workloads are seeded uniform integers.

Paged decode inputs: per sequence b, its L_b cached tokens are drawn like K
and V (one (L_b, Hkv, d) slice each, N(0, 1) rounded to bf16) and written
into pages of a cache whose physical pages are a seeded random permutation
(so consecutive pages of a sequence are scattered); pages that no sequence
uses hold N(0, 1) values too.  The queries (B, Hq, T, d) are drawn the same
way.  Context lengths for the workloads are seeded uniform integers in
[1, max_len] (``decode_lengths``).
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


def make_packed_qkv(lens, Hq: int, Hkv: int, d: int, seed: int):
    """Packed sequences: bf16 CPU tensors q (Hq, total, d), k and v
    (Hkv, total, d), and cu_seqlens (B + 1,) int32; each head's rows drawn as
    one (total, d) slice, in the order Q, K, V."""
    total = int(sum(lens))
    gen = torch.Generator().manual_seed(int(seed))
    q = _draw(gen, 1, Hq, total, d)[0]
    k = _draw(gen, 1, Hkv, total, d)[0]
    v = _draw(gen, 1, Hkv, total, d)[0]
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)
    return q, k, v, cu


def decode_lengths(B: int, max_len: int, seed: int) -> list[int]:
    """Seeded context lengths, uniform in [1, max_len]."""
    rng = np.random.default_rng(int(seed))
    return [int(x) for x in rng.integers(1, max_len + 1, size=B)]


def make_paged_kv(lens, Hkv: int, d: int, page_size: int, seed: int, extra_pages: int = 2):
    """Return (k_cache, v_cache, block_table) as CPU tensors.

    k_cache, v_cache: bf16 (num_pages, page_size, Hkv, d); block_table:
    int32 (B, max_pages) with max_pages = max ceil(L_b / page_size) (at least
    1); entries past a sequence's pages are -1.
    """
    gen = torch.Generator().manual_seed(int(seed))
    rng = np.random.default_rng(int(seed) + 1)
    npg = [(int(L) + page_size - 1) // page_size for L in lens]
    num_pages = sum(npg) + extra_pages
    max_pages = max(max(npg), 1)
    perm = rng.permutation(num_pages)
    kc = torch.empty((num_pages, page_size, Hkv, d), dtype=torch.bfloat16)
    vc = torch.empty_like(kc)
    table = torch.full((len(lens), max_pages), -1, dtype=torch.int32)
    used = np.zeros(num_pages, dtype=bool)
    nxt = 0
    for b, L in enumerate(lens):
        k = torch.randn((int(L), Hkv, d), generator=gen, dtype=torch.float32).to(torch.bfloat16)
        v = torch.randn((int(L), Hkv, d), generator=gen, dtype=torch.float32).to(torch.bfloat16)
        for p in range(npg[b]):
            page = int(perm[nxt])
            nxt += 1
            used[page] = True
            table[b, p] = page
            n = min(page_size, int(L) - p * page_size)
            kc[page, :n] = k[p * page_size:p * page_size + n]
            vc[page, :n] = v[p * page_size:p * page_size + n]
            if n < page_size:
                kc[page, n:] = torch.randn((page_size - n, Hkv, d), generator=gen).to(torch.bfloat16)
                vc[page, n:] = torch.randn((page_size - n, Hkv, d), generator=gen).to(torch.bfloat16)
    for page in np.nonzero(~used)[0]:
        kc[page] = torch.randn((page_size, Hkv, d), generator=gen).to(torch.bfloat16)
        vc[page] = torch.randn((page_size, Hkv, d), generator=gen).to(torch.bfloat16)
    return kc, vc, table


def make_decode_q(B: int, Hq: int, T: int, d: int, seed: int) -> torch.Tensor:
    """Return bf16 queries (B, Hq, T, d)."""
    gen = torch.Generator().manual_seed(int(seed))
    return _draw(gen, B, Hq, T, d)


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
