"""Pins for the paged-decode oracle (no GPU).

The decode oracle gathers K and V through a page table and applies the plain
definition.  It is tied to the separately pinned forward oracle (the same
tokens stored contiguously, the same query rows), to the pure-Python brute
force, to invariants of the paging (any page permutation, shared pages) and
to closed forms; the merge rule is tied to the unsplit result.  Planted
mistakes in the gather must be caught.
"""

import math

import numpy as np
import pytest

from oracle import attention_forward, brute_attention, decode_paged, merge_partials
from oracle import decode as oracle_decode


def _paged_from_contiguous(k, v, lens, ps, seed, extra_pages=3):
    """Store contiguous (B, Hkv, N, d) K/V into a shuffled paged cache.

    Returns k_cache, v_cache (num_pages, ps, Hkv, d) and block_table (B, maxp)
    whose rows point at distinct random physical pages; unused slots hold
    garbage so that a wrong gather shows.
    """
    rng = np.random.default_rng(seed)
    B, Hkv, N, d = k.shape
    maxp = (N + ps - 1) // ps
    need = sum((L + ps - 1) // ps for L in lens)
    num_pages = need + extra_pages
    perm = rng.permutation(num_pages)
    kc = rng.standard_normal((num_pages, ps, Hkv, d)) * 100.0
    vc = rng.standard_normal((num_pages, ps, Hkv, d)) * 100.0
    table = rng.integers(0, num_pages, size=(B, maxp))
    nxt = 0
    for b, L in enumerate(lens):
        for p in range((L + ps - 1) // ps):
            page = perm[nxt]
            nxt += 1
            table[b, p] = page
            n = min(ps, L - p * ps)
            kc[page, :n] = np.transpose(k[b, :, p * ps:p * ps + n], (1, 0, 2))
            vc[page, :n] = np.transpose(v[b, :, p * ps:p * ps + n], (1, 0, 2))
    return kc, vc, table


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("window", [0, 1, 5, 40])
@pytest.mark.parametrize("Hq,Hkv,T", [(2, 2, 1), (4, 1, 1), (6, 2, 3), (8, 8, 4)])
def test_matches_forward_oracle_on_the_contiguous_cache(window, Hq, Hkv, T):
    B, N, d, ps = 3, 45, 16, 8
    lens = [45, 17, 8]
    q_full = _rand((B, Hq, N, d), 1)
    k, v = _rand((B, Hkv, N, d), 2), _rand((B, Hkv, N, d), 3)
    kc, vc, table = _paged_from_contiguous(k, v, lens, ps, seed=4)
    q = np.stack([q_full[b, :, L - T:L] for b, L in enumerate(lens)])
    o, lse = decode_paged(q, kc, vc, table, lens, 0.3, window)
    for b, L in enumerate(lens):
        of, lf = attention_forward(q_full[b:b + 1, :, :L], k[b:b + 1, :, :L], v[b:b + 1, :, :L],
                                   0.3, True, window)
        np.testing.assert_allclose(o[b], of[0, :, L - T:L], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[b], lf[0, :, L - T:L], rtol=0, atol=1e-13)


def test_matches_brute_force():
    B, Hq, Hkv, N, d, ps, T = 2, 4, 2, 11, 3, 4, 2
    lens = [11, 6]
    q_full = _rand((B, Hq, N, d), 5)
    k, v = _rand((B, Hkv, N, d), 6), _rand((B, Hkv, N, d), 7)
    kc, vc, table = _paged_from_contiguous(k, v, lens, ps, seed=8)
    q = np.stack([q_full[b, :, L - T:L] for b, L in enumerate(lens)])
    o, lse = decode_paged(q, kc, vc, table, lens, 0.8, 3)
    for b, L in enumerate(lens):
        ob, lb = brute_attention(q_full[b:b + 1, :, :L].tolist(), k[b:b + 1, :, :L].tolist(),
                                 v[b:b + 1, :, :L].tolist(), 0.8, True, 3)
        np.testing.assert_allclose(o[b], np.array(ob)[0, :, L - T:L], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b], np.array(lb)[0, :, L - T:L], rtol=0, atol=1e-12)


def test_page_permutation_and_shared_pages():
    rng = np.random.default_rng(9)
    num_pages, ps, Hkv, d = 12, 4, 2, 8
    kc, vc = rng.standard_normal((num_pages, ps, Hkv, d)), rng.standard_normal((num_pages, ps, Hkv, d))
    table = np.array([[3, 7, 1, 0], [3, 7, 5, 2]])  # both sequences share pages 3 and 7
    lens = [10, 16]
    q = rng.standard_normal((2, 4, 1, d))
    q[1] = q[0]
    o, lse = decode_paged(q, kc, vc, table, [8, 8], 0.5)
    # the same 8 shared tokens and the same query give the same answer
    np.testing.assert_array_equal(o[0], o[1])
    np.testing.assert_array_equal(lse[0], lse[1])
    # relabelling physical pages changes nothing
    perm = rng.permutation(num_pages)
    inv = np.argsort(perm)
    o1, l1 = decode_paged(q, kc, vc, table, lens, 0.5)
    o2, l2 = decode_paged(q, kc[inv], vc[inv], perm[table], lens, 0.5)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_closed_forms():
    num_pages, ps, d = 4, 4, 5
    rng = np.random.default_rng(10)
    kc, vc = rng.standard_normal((num_pages, ps, 1, d)), rng.standard_normal((num_pages, ps, 1, d))
    q = rng.standard_normal((1, 1, 1, d))
    table = np.array([[2, 0, 1, 3]])
    # one cached token: o = v, lse = sigma q.k
    o, lse = decode_paged(q, kc, vc, table, [1], 0.25)
    np.testing.assert_allclose(o[0, 0, 0], vc[2, 0, 0], rtol=0, atol=1e-15)
    assert math.isclose(lse[0, 0, 0], 0.25 * float(q[0, 0, 0] @ kc[2, 0, 0]), abs_tol=1e-14)
    # q = 0: uniform weights over the window: lse = ln w, o = mean of the last w values
    o, lse = decode_paged(np.zeros((1, 1, 1, d)), kc, vc, table, [13], 1.0, window=6)
    toks = np.concatenate([vc[p, :, 0] for p in table[0]])[:13]
    np.testing.assert_allclose(o[0, 0, 0], toks[7:13].mean(0), rtol=0, atol=1e-14)
    assert math.isclose(lse[0, 0, 0], math.log(6), abs_tol=1e-14)
    # more queries than cached tokens: the first query sees nothing
    o, lse = decode_paged(rng.standard_normal((1, 1, 3, d)), kc, vc, table, [2], 1.0)
    assert lse[0, 0, 0] == -np.inf and not o[0, 0, 0].any()
    assert np.isfinite(lse[0, 0, 1:]).all()


def test_merge_of_disjoint_key_ranges_equals_the_whole():
    rng = np.random.default_rng(11)
    num_pages, ps, Hkv, d = 10, 8, 2, 16
    kc, vc = rng.standard_normal((num_pages, ps, Hkv, d)), rng.standard_normal((num_pages, ps, Hkv, d))
    table = np.array([[4, 9, 0, 6, 2, 7]])
    q = rng.standard_normal((1, 4, 1, d)) * 2
    L = 45
    o, lse = decode_paged(q, kc, vc, table, [L], 0.7)
    parts_o, parts_l = [], []
    # key ranges [0, 16), [16, 40), [40, 45) plus an empty part
    for p0, p1 in ((0, 2), (2, 5), (5, 6)):
        n = min(L, p1 * ps) - p0 * ps
        po, pl = decode_paged(q, kc, vc, table[:, p0:p1], [n], 0.7)
        parts_o.append(po)
        parts_l.append(pl)
    parts_o.append(np.zeros_like(o))
    parts_l.append(np.full_like(lse, -np.inf))
    mo, ml = merge_partials(parts_o, parts_l)
    np.testing.assert_allclose(mo, o, rtol=0, atol=1e-14)
    np.testing.assert_allclose(ml, lse, rtol=0, atol=1e-13)
    # all parts empty: o = 0, lse = -inf
    eo, el = merge_partials([np.zeros_like(o)] * 2, [np.full_like(lse, -np.inf)] * 2)
    assert not eo.any() and (el == -np.inf).all()


def test_planted_gather_mistakes_are_caught(monkeypatch):
    real = oracle_decode.gather_pages

    def off_by_one_slot(cache, table_row, length):
        ps = cache.shape[1]
        j = np.arange(length)
        return cache[np.asarray(table_row)[j // ps], (j + 1) % ps]

    def fails():
        try:
            test_matches_forward_oracle_on_the_contiguous_cache(0, 4, 2, 1)
        except AssertionError:
            return True
        return False

    assert not fails()
    monkeypatch.setattr(oracle_decode, "gather_pages", off_by_one_slot)
    assert fails()
    monkeypatch.setattr(oracle_decode, "gather_pages", real)


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        decode_paged(np.zeros((1, 3, 1, 4)), np.zeros((2, 4, 2, 4)), np.zeros((2, 4, 2, 4)),
                     np.zeros((1, 1), dtype=int), [1], 1.0)
    with pytest.raises(ValueError):
        decode_paged(np.zeros((1, 2, 1, 4)), np.zeros((2, 4, 2, 4)), np.zeros((2, 4, 2, 4)),
                     np.zeros((1, 1), dtype=int), [9], 1.0)
