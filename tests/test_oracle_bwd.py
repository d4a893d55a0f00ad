"""Pins for the gradient oracle (no GPU).

Each check ties ``oracle.attention_backward`` to something other than its own
formulas: central finite differences of the (separately pinned) forward
oracle, float64 autograd through torch's scaled_dot_product_attention with an
explicit mask, closed forms of special cases, and the GQA reduction.  The
last group plants mistakes and checks that the pins notice.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention_backward, attention_forward
from oracle import backward as oracle_backward

MASKS = [(False, 0), (True, 0), (True, 1), (True, 2), (True, 4)]


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _loss(q, k, v, do, scale, causal, window):
    o, _ = attention_forward(q, k, v, scale, causal, window)
    return float(np.sum(o * do))


def _finite_difference(q, k, v, do, scale, causal, window, h=1e-6):
    """Central differences of sum(O * do) for every input element."""
    grads = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        x = args[which]
        g = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(*args, do, scale, causal, window)
            x[idx] = old - h
            lm = _loss(*args, do, scale, causal, window)
            x[idx] = old
            g[idx] = (lp - lm) / (2 * h)
        grads.append(g)
    return grads


@pytest.mark.parametrize("causal,window", MASKS)
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (2, 1), (3, 1)])
def test_gradients_match_finite_differences(causal, window, Hq, Hkv):
    N, d = 5, 3
    q = _rand((1, Hq, N, d), 11)
    k = _rand((1, Hkv, N, d), 12)
    v = _rand((1, Hkv, N, d), 13)
    do = _rand((1, Hq, N, d), 14)
    scale = 0.7
    dq, dk, dv = attention_backward(q, k, v, do, scale, causal, window, block=2)
    fq, fk, fv = _finite_difference(q, k, v, do, scale, causal, window)
    for got, want in ((dq, fq), (dk, fk), (dv, fv)):
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-7)


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 7), (True, 64)])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 2), (4, 1)])
def test_gradients_match_torch_autograd_float64(causal, window, Hq, Hkv):
    N, d = 40, 16
    q = _rand((2, Hq, N, d), 21)
    k = _rand((2, Hkv, N, d), 22)
    v = _rand((2, Hkv, N, d), 23)
    do = _rand((2, Hq, N, d), 24)
    scale = 1 / math.sqrt(d)
    G = Hq // Hkv
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    i = torch.arange(N)[:, None]
    j = torch.arange(N)[None, :]
    allowed = torch.ones(N, N, dtype=torch.bool)
    if causal:
        allowed &= j <= i
    if window > 0:
        allowed &= j > i - window
    o = F.scaled_dot_product_attention(tq, tk.repeat_interleave(G, dim=1),
                                       tv.repeat_interleave(G, dim=1), attn_mask=allowed,
                                       scale=float(np.float32(scale)))
    (o * torch.tensor(do)).sum().backward()
    dq, dk, dv = attention_backward(q, k, v, do, scale, causal, window, block=16)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-11)


@pytest.mark.parametrize("causal,window", MASKS)
def test_constant_v_has_no_query_or_key_gradient(causal, window):
    # O = c for every row whatever Q and K are, so dQ = dK = 0
    N, d = 12, 4
    q, k = _rand((1, 2, N, d), 31), _rand((1, 2, N, d), 32)
    v = np.broadcast_to(np.array([0.5, -1.25, 2.0, 0.0]), (1, 2, N, d)).copy()
    do = _rand((1, 2, N, d), 33)
    dq, dk, dv = attention_backward(q, k, v, do, 0.4, causal, window)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    assert np.abs(dv).max() > 0.1


@pytest.mark.parametrize("causal,window", MASKS)
def test_zero_query_gives_uniform_value_gradient(causal, window):
    # Q = 0: row i weights its |V_i| visible keys equally, so
    # dV_j = sum over the rows i that see j of dO_i / |V_i|
    N, d = 9, 3
    q = np.zeros((1, 1, N, d))
    k, v = _rand((1, 1, N, d), 41), _rand((1, 1, N, d), 42)
    do = _rand((1, 1, N, d), 43)
    _, _, dv = attention_backward(q, k, v, do, 1.3, causal, window)
    want = np.zeros((N, d))
    for i in range(N):
        vis = [j for j in range(N) if (not causal or j <= i) and (window <= 0 or j > i - window)]
        for j in vis:
            want[j] += do[0, 0, i] / len(vis)
    np.testing.assert_allclose(dv[0, 0], want, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 3)])
def test_gqa_gradients_sum_over_the_group(causal, window):
    N, d, Hq, Hkv = 10, 4, 6, 2
    G = Hq // Hkv
    q, do = _rand((1, Hq, N, d), 51), _rand((1, Hq, N, d), 52)
    k, v = _rand((1, Hkv, N, d), 53), _rand((1, Hkv, N, d), 54)
    dq, dk, dv = attention_backward(q, k, v, do, 0.5, causal, window)
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    dq2, dk2, dv2 = attention_backward(q, kr, vr, do, 0.5, causal, window)
    np.testing.assert_allclose(dq, dq2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk, dk2.reshape(1, Hkv, G, N, d).sum(2), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv, dv2.reshape(1, Hkv, G, N, d).sum(2), rtol=0, atol=1e-13)


def test_threaded_equals_serial():
    q, do = _rand((2, 4, 33, 8), 61), _rand((2, 4, 33, 8), 62)
    k, v = _rand((2, 2, 33, 8), 63), _rand((2, 2, 33, 8), 64)
    a = attention_backward(q, k, v, do, 0.3, True, 9, block=5)
    b = attention_backward(q, k, v, do, 0.3, True, 9, block=5, workers=4)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_rejects_mismatched_upstream_gradient():
    q = np.zeros((1, 1, 4, 2))
    with pytest.raises(ValueError):
        attention_backward(q, q, q, np.zeros((1, 1, 4, 3)), 1.0)


# --------------------------------------------------------------------------
# planted mistakes must be caught by the finite-difference pin
# --------------------------------------------------------------------------

def _fd_pin_fails():
    N, d = 4, 2
    q, k, v = _rand((1, 2, N, d), 71), _rand((1, 1, N, d), 72), _rand((1, 1, N, d), 73)
    do = _rand((1, 2, N, d), 74)
    got = attention_backward(q, k, v, do, 0.9, True, 0)
    want = _finite_difference(q, k, v, do, 0.9, True, 0)
    return any(not np.allclose(g, w, rtol=0, atol=1e-7) for g, w in zip(got, want))


def test_planted_missing_delta_is_caught(monkeypatch):
    real = np.einsum

    def no_delta(spec, a, b):
        return np.zeros(a.shape[0]) if spec == "ij,ij->i" else real(spec, a, b)

    monkeypatch.setattr(oracle_backward.np, "einsum", no_delta)
    assert _fd_pin_fails()


def test_planted_transposed_probabilities_are_caught(monkeypatch):
    real = oracle_backward.rows_probabilities

    def transposed(qh, kh, rows, sigma, causal, window, N):
        p, lo, hi, lse = real(qh, kh, rows, sigma, causal, window, N)
        if p.shape[0] == p.shape[1]:
            p = p.T.copy()
        return p, lo, hi, lse

    monkeypatch.setattr(oracle_backward, "rows_probabilities", transposed)
    assert _fd_pin_fails()


def test_planted_wrong_scale_is_caught(monkeypatch):
    real = oracle_backward.rows_probabilities

    def doubled(qh, kh, rows, sigma, causal, window, N):
        return real(qh, kh, rows, 2 * sigma, causal, window, N)

    monkeypatch.setattr(oracle_backward, "rows_probabilities", doubled)
    assert _fd_pin_fails()
