"""Pins for the packed-sequence / structured-mask oracle (no GPU).

Tied to the separately pinned forward oracle (each packed sequence alone,
masks without band or global tokens), to a per-pair brute force written
here with math.fsum over the rule evaluated pair by pair, and to closed
forms; planted mistakes must be caught.

The visibility rule itself (local band plus global tokens, combined with a
causal mask or a causal sliding window: "Efficient attention: long context
and sub-quadratic variants", section "Sliding-window and local attention";
"Efficient Attention: FlashAttention, Sparse, Linear", section 45.2.2) is
pinned by visible-key sets written out by hand below, which call nothing in
the oracle: a global row is limited only by the causal mask, every row sees
the global keys it is causally allowed to see, and the window and the band
cut only non-global pairs.
"""

import math

import numpy as np
import pytest

from oracle import attention_forward, attention_general, visible
from oracle import general as oracle_general

RULES = [  # causal, window, radius, n_global
    (False, 0, 0, 0), (True, 0, 0, 0), (True, 7, 0, 0),
    (False, 0, 3, 0), (False, 0, 3, 2), (True, 0, 4, 3), (True, 5, 2, 1), (False, 0, 0, 4),
]


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _brute(q, k, v, scale, cu, causal, window, radius, n_global):
    Hq, total, d = q.shape
    G = Hq // k.shape[0]
    sigma = float(np.float32(scale))
    o = np.zeros_like(q)
    lse = np.zeros((Hq, total))
    for h in range(Hq):
        for b in range(len(cu) - 1):
            s0, N = cu[b], cu[b + 1] - cu[b]
            for i in range(N):
                sc = {j: sigma * math.fsum(q[h, s0 + i, t] * k[h // G, s0 + j, t] for t in range(d))
                      for j in range(N) if visible(i, j, causal, window, radius, n_global)}
                top = max(sc.values())
                w = {j: math.exp(x - top) for j, x in sc.items()}
                den = math.fsum(w.values())
                for t in range(d):
                    o[h, s0 + i, t] = math.fsum(w[j] * v[h // G, s0 + j, t] for j in w) / den
                lse[h, s0 + i] = top + math.log(den)
    return o, lse


@pytest.mark.parametrize("rule", RULES)
def test_matches_brute_force(rule):
    causal, window, radius, n_global = rule
    cu = [0, 9, 10, 23]
    q, k, v = _rand((4, 23, 3), 1), _rand((2, 23, 3), 2), _rand((2, 23, 3), 3)
    o, lse = attention_general(q, k, v, 0.6, cu, causal, window, radius, n_global, block=4)
    ob, lb = _brute(q, k, v, 0.6, cu, causal, window, radius, n_global)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 17)])
def test_packed_sequences_match_the_forward_oracle_one_by_one(causal, window):
    cu = [0, 100, 101, 300, 364]
    Hq, Hkv, d = 6, 2, 8
    q, k, v = _rand((Hq, 364, d), 4), _rand((Hkv, 364, d), 5), _rand((Hkv, 364, d), 6)
    o, lse = attention_general(q, k, v, 0.4, cu, causal, window, block=32, workers=3)
    for a, b in zip(cu, cu[1:]):
        of, lf = attention_forward(q[None, :, a:b], k[None, :, a:b], v[None, :, a:b], 0.4, causal,
                                   window)
        np.testing.assert_allclose(o[:, a:b], of[0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[:, a:b], lf[0], rtol=0, atol=1e-13)


def test_closed_forms():
    N, d = 40, 5
    k, v = _rand((1, N, d), 7), _rand((1, N, d), 8)
    q = np.zeros((1, N, d))
    # Q = 0: uniform weights over each row's visible set
    o, lse = attention_general(q, k, v, 1.0, [0, N], False, 0, 3, 2)
    for i in range(N):
        vis = [j for j in range(N) if visible(i, j, False, 0, 3, 2)]
        np.testing.assert_allclose(o[0, i], v[0, vis].mean(0), rtol=0, atol=1e-13)
        assert math.isclose(lse[0, i], math.log(len(vis)), abs_tol=1e-13)
    # global rows see everything; a row far from the globals sees 2 + 7 keys
    assert len([j for j in range(N) if visible(0, j, False, 0, 3, 2)]) == N
    assert len([j for j in range(N) if visible(20, j, False, 0, 3, 2)]) == 2 + 7


def test_planted_mistakes_are_caught(monkeypatch):
    real = oracle_general._candidate_keys

    def band_too_narrow(r0, r1, N, causal, window, radius, n_global):
        keys = real(r0, r1, N, causal, window, radius, n_global)
        return keys[keys >= min(n_global, 1)] if n_global else keys  # drops global key 0

    cu = [0, 23]
    q, k, v = _rand((1, 23, 3), 9), _rand((1, 23, 3), 10), _rand((1, 23, 3), 11)
    ob, _ = _brute(q, k, v, 0.6, cu, False, 0, 3, 2)
    monkeypatch.setattr(oracle_general, "_candidate_keys", band_too_narrow)
    o, _ = attention_general(q, k, v, 0.6, cu, False, 0, 3, 2, block=4)
    assert not np.allclose(o, ob, atol=1e-6)


def test_rejects_bad_input():
    z = np.zeros((1, 4, 2))
    with pytest.raises(ValueError):
        attention_general(z, z, z, 1.0, [0, 3])
    with pytest.raises(ValueError):
        attention_general(z, z, z, 1.0, [0, 3, 2, 4])
    with pytest.raises(ValueError):
        attention_general(z, z, z, 1.0, [0, 4], causal=False, window=2)


# Visible keys written out by hand for N = 12 (one sequence), per rule
# (causal, window, radius, n_global): row -> sorted key list.
N_HAND = 12
HAND = {
    (True, 0, 0, 3): {
        1: [0, 1],                        # global row: causal only
        2: [0, 1, 2],
        3: [0, 1, 2, 3],                  # first non-global row
        10: list(range(11)),
    },
    (True, 5, 0, 2): {
        1: [0, 1],
        2: [0, 1, 2],
        6: [0, 1, 2, 3, 4, 5, 6],         # window 2..6 plus the globals
        7: [0, 1, 3, 4, 5, 6, 7],         # key 2 falls out of the window
        11: [0, 1, 7, 8, 9, 10, 11],      # past the window: globals stay
    },
    (True, 2, 0, 4): {
        3: [0, 1, 2, 3],                  # global row wider than the window
        4: [0, 1, 2, 3, 4],
        9: [0, 1, 2, 3, 8, 9],
    },
    (True, 0, 2, 1): {
        0: [0],
        1: [0, 1],
        3: [0, 1, 2, 3],
        8: [0, 6, 7, 8],                  # past the band: global key 0 stays
    },
    (False, 0, 0, 4): {
        0: list(range(12)),
        4: list(range(12)),
        11: list(range(12)),
    },
    (False, 0, 2, 2): {
        0: list(range(12)),               # global row sees everything
        1: list(range(12)),
        2: [0, 1, 2, 3, 4],
        9: [0, 1, 7, 8, 9, 10, 11],
        11: [0, 1, 9, 10, 11],
    },
}


@pytest.mark.parametrize("rule", sorted(HAND))
def test_visible_sets_match_the_hand_written_lists(rule):
    causal, window, radius, n_global = rule
    jj = np.arange(N_HAND)
    for i, keys in HAND[rule].items():
        assert [j for j in range(N_HAND) if visible(i, j, *rule)] == keys, (rule, i)
        mask = oracle_general.visible_block(np.int64(i), jj, causal, window, radius, n_global)
        assert list(np.flatnonzero(mask)) == keys, (rule, i)


def _q_zero_errors(block):
    """Largest deviation of the oracle from the Q = 0 closed form (uniform
    weights over the hand-written visible set: o = mean of those V rows,
    lse = log of their count) over every rule and listed row; two packed
    sequences of N_HAND rows, so the offsets of the second are exercised."""
    cu = [0, N_HAND, 2 * N_HAND]
    v = _rand((1, 2 * N_HAND, 4), 21)
    k = _rand((1, 2 * N_HAND, 4), 22)
    q = np.zeros((1, 2 * N_HAND, 4))
    worst = 0.0
    for rule, rows in HAND.items():
        causal, window, radius, n_global = rule
        o, lse = attention_general(q, k, v, 0.9, cu, causal, window, radius, n_global,
                                   block=block)
        for s0 in cu[:-1]:
            for i, keys in rows.items():
                want = v[0, [s0 + j for j in keys]].mean(0)
                worst = max(worst, float(np.abs(o[0, s0 + i] - want).max()),
                            abs(float(lse[0, s0 + i]) - math.log(len(keys))))
    return worst


@pytest.mark.parametrize("block", [4, 128])
def test_q_zero_closed_forms_from_the_hand_written_lists(block):
    assert _q_zero_errors(block) <= 1e-13


def _window_on_global_keys(i, j, causal=False, window=0, radius=0, n_global=0):
    vis = np.ones(np.broadcast(i, j).shape, dtype=bool)
    if causal:
        vis &= j <= i
    if window > 0:
        vis &= (i < n_global) | (j > i - window)
    if radius > 0:
        vis &= (i < n_global) | (j < n_global) | (np.abs(i - j) <= radius)
    return vis


def _window_on_global_rows(i, j, causal=False, window=0, radius=0, n_global=0):
    vis = np.ones(np.broadcast(i, j).shape, dtype=bool)
    if causal:
        vis &= j <= i
    if window > 0:
        vis &= j > i - window
    if radius > 0:
        vis &= (i < n_global) | (j < n_global) | (np.abs(i - j) <= radius)
    return vis


def _causal_global_sees_later_keys(i, j, causal=False, window=0, radius=0, n_global=0):
    local = np.ones(np.broadcast(i, j).shape, dtype=bool)
    if causal:
        local &= j <= i
    if window > 0:
        local &= j > i - window
    if radius > 0:
        local &= np.abs(i - j) <= radius
    return (i < n_global) | (local | ((j < n_global) & (j <= i if causal else True)))


def _band_not_symmetric(i, j, causal=False, window=0, radius=0, n_global=0):
    vis = np.ones(np.broadcast(i, j).shape, dtype=bool)
    if causal:
        vis &= j <= i
    local = np.ones_like(vis)
    if window > 0:
        local &= j > i - window
    if radius > 0:
        local &= (i - j <= radius) & (j <= i)
    return vis & ((i < n_global) | (j < n_global) | local)


@pytest.mark.parametrize("mistake", [_window_on_global_keys, _window_on_global_rows,
                                     _causal_global_sees_later_keys, _band_not_symmetric])
def test_planted_rule_mistakes_fail_the_hand_written_pins(monkeypatch, mistake):
    monkeypatch.setattr(oracle_general, "visible_block", mistake)
    assert _q_zero_errors(128) > 1e-3
