"""Pins for the FP8 quantisation oracle (no GPU): the OCP E4M3 table's
closed-form values, rounding against a brute-force nearest search over all
codes and against torch's float8_e4m3fn conversion, the power-of-two scale's
defining property, and planted rounding mistakes."""

import math

import numpy as np
import pytest
import torch

from oracle import fp8 as F


def test_decode_closed_forms():
    d = F.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert d[0x00] == 0.0 and np.signbit(d[0x80])
    assert d[0x01] == 2.0 ** -9 and d[0x07] == 7 * 2.0 ** -9       # subnormals
    assert d[0x08] == 2.0 ** -6                                      # smallest normal
    assert d[0x38] == 1.0 and d[0x3F] == 1.875 and d[0x40] == 2.0
    assert d[0x7E] == 448.0 and d[0xFE] == -448.0
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])
    pos = d[:0x7F]
    assert np.all(np.diff(pos) > 0)                                  # codes are ordered
    assert np.array_equal(d[0x80:0xFF], -d[:0x7F])


def test_encode_decode_round_trip():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(F.e4m3_encode(F.e4m3_decode(codes)), codes)


def _nearest_brute(x):
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = F.e4m3_decode(codes)
    out = np.empty_like(x)
    for i, xi in enumerate(x):
        dist = np.abs(vals - xi)
        best = np.flatnonzero(dist == dist.min())
        even = [b for b in best if codes[b] % 2 == 0]   # ties: the even mantissa
        out[i] = vals[even[0] if even else best[0]]
    return out


def test_rounding_matches_brute_force_including_ties():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.uniform(-448, 448, 3000), rng.uniform(-1, 1, 3000) * 2.0 ** -5,
                        rng.normal(size=2000)])
    # exact ties: midpoints between neighbouring codes
    vals = np.sort(F.e4m3_decode(np.arange(0x7E, dtype=np.uint8)))
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([x, mids, -mids])
    got = F.e4m3_round(x)
    want = _nearest_brute(x)
    assert np.array_equal(np.abs(got), np.abs(want))


def test_rounding_matches_torch_float8_e4m3fn():
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch without float8_e4m3fn")
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.uniform(-448, 448, 20000), rng.normal(size=20000) * 1e-2])
    t = torch.tensor(x, dtype=torch.float32).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(F.e4m3_round(x.astype(np.float32).astype(np.float64)), t)


@pytest.mark.parametrize("amax,want", [(448.0, 1.0), (448.0001, 2.0), (449.0, 2.0),
                                       (224.0, 0.5), (224.5, 1.0), (1.0, 2.0 ** -8),
                                       (1.75, 2.0 ** -8), (1.76, 2.0 ** -7), (0.0, 1.0)])
def test_pow2_scale_cases(amax, want):
    assert F.pow2_scale(amax) == want


def test_pow2_scale_property():
    rng = np.random.default_rng(3)
    for a in np.exp(rng.uniform(-30, 30, 2000)):
        s = F.pow2_scale(a)
        assert math.log2(s) == int(math.log2(s))
        assert a <= 448 * s and a > 448 * s / 2


def test_quantize_never_saturates_and_is_within_half_an_ulp():
    rng = np.random.default_rng(4)
    x = rng.normal(size=(3, 50)) * 7.3
    codes, s, deq = F.quantize(x)
    assert np.all(np.abs(x / s) <= 448)
    assert np.array_equal(F.e4m3_decode(codes) * s, deq)
    rel = np.abs(deq - x) / np.maximum(np.abs(x), 2.0 ** -6 * s)
    assert rel.max() <= 2.0 ** -4 + 1e-12


def test_planted_round_half_away_is_caught(monkeypatch):
    def half_away(x):
        x = np.asarray(x, dtype=np.float64)
        mag = np.abs(x)
        e = np.maximum(np.floor(np.log2(np.where(mag > 0, mag, 1.0))), -6)
        ulp = np.exp2(e - 3)
        return np.copysign(np.floor(mag / ulp + 0.5) * ulp, x)
    vals = np.sort(F.e4m3_decode(np.arange(0x7E, dtype=np.uint8)))
    mids = (vals[:-1] + vals[1:]) / 2
    assert not np.array_equal(np.abs(half_away(mids)), np.abs(_nearest_brute(mids)))
