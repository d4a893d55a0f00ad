"""FP8 (OCP e4m3) quantisation and the attention it feeds -- TEST
INFRASTRUCTURE ONLY: see the package docstring for who may import this.

"Efficient attention: long context and sub-quadratic variants" attaches an
FP8 path to FlashAttention-3 (section "FlashAttention: exact attention,
IO-aware") but fixes no format or scaling.  Reading 16:

* format: OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7,
  3 mantissa bits; exponent field 0 holds the subnormals m/8 * 2^-6; the
  all-ones exponent with all-ones mantissa is NaN; there are no infinities;
  the largest finite value is 1.75 * 2^8 = 448.  Rounding to nearest, ties
  to even.
* per-tensor scales that are powers of two: for a tensor with largest
  magnitude amax, s = 2^e with e the smallest integer such that
  amax <= 448 * 2^e (e = 0 for an all-zero tensor), so x / s is exact in
  fp32 and never saturates; the code of x is e4m3(x / s) and its value
  code * s.
* the attention is the plain definition applied to the dequantised Q, K, V
  (codes times scales); the FP8 kernel's own rounding of the weights P to
  e4m3 before the P V product is an approximation whose error the GPU
  tolerance accounts for.

Functions: ``e4m3_round`` (values), ``e4m3_encode`` / ``e4m3_decode``
(bytes), ``pow2_scale``, ``quantize``, ``fp8_attention_reference``.
"""

from __future__ import annotations

import math

import numpy as np

from .attention import attention_forward

E4M3_MAX = 448.0
_MIN_NORMAL_EXP = -6
_MANT_BITS = 3


def e4m3_round(x):
    """Round float64 values to the nearest e4m3 value (ties to even).

    Values must satisfy |x| <= 448 (the callers' scaling guarantees it)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("|x| > 448 cannot be represented")
    mag = np.abs(x)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
    e = np.maximum(e, _MIN_NORMAL_EXP)          # subnormals share the 2^-6 binade's step
    ulp = np.exp2(e - _MANT_BITS)
    r = np.round(mag / ulp) * ulp                # np.round: half to even
    return np.copysign(r, x)


def e4m3_decode(codes):
    """Byte codes (uint8) -> float64 values (NaN for the NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return s * val


def e4m3_encode(x):
    """Float values already on the e4m3 grid -> byte codes (the sign of zero
    kept)."""
    x = np.asarray(x, dtype=np.float64)
    mag = np.abs(x)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
    normal = mag >= 2.0 ** -6
    ef = np.where(normal, e + 7, 0).astype(np.int64)
    m = np.where(normal, mag / np.exp2(e) - 1.0, mag / 2.0 ** -6) * 8.0
    mi = np.rint(m).astype(np.int64)
    if np.any(np.abs(m - mi) > 1e-9) or np.any(mag > E4M3_MAX):
        raise ValueError("value not on the e4m3 grid")
    sign = np.signbit(x).astype(np.int64)
    return ((sign << 7) | (ef << 3) | mi).astype(np.uint8)


def pow2_scale(amax: float) -> float:
    """2^e for the smallest integer e with amax <= 448 * 2^e (1.0 for 0)."""
    amax = float(amax)
    if amax == 0.0:
        return 1.0
    f, E = math.frexp(amax)   # amax = f * 2^E, 0.5 <= f < 1; 448 = 0.875 * 2^9
    e = E - 9 if f <= 0.875 else E - 8
    return math.ldexp(1.0, e)


def quantize(x):
    """Per-tensor FP8 quantisation: returns (codes uint8, scale, dequantised)."""
    x = np.asarray(x, dtype=np.float64)
    s = pow2_scale(np.abs(x).max() if x.size else 0.0)
    v = e4m3_round(x / s)
    return e4m3_encode(v), s, v * s


def fp8_attention_reference(q, k, v, scale, causal=False, window=0, workers=1):
    """Quantise q, k, v per tensor and return the exact attention of the
    dequantised tensors: (o, lse, (codes_q, codes_k, codes_v),
    (s_q, s_k, s_v))."""
    cq, sq, dq = quantize(q)
    ck, sk, dk = quantize(k)
    cv, sv, dv = quantize(v)
    o, lse = attention_forward(dq, dk, dv, scale, causal, window, workers=workers)
    return o, lse, (cq, ck, cv), (sq, sk, sv)
