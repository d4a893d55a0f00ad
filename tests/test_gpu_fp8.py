"""GPU parity of the FP8 path (attn_fp8_quantize + attn_fwd_fp8) against the
FP8 oracle.

* Codes and scales: bit-exact (the per-tensor scales are powers of two, so
  x / s is exact and both sides round the same fp32 value to nearest even).
* Attention: against the exact float64 attention of the dequantised tensors.
  The kernel rounds each weight P (scaled to at most 2^8) to e4m3 before the
  P V product: a relative error of at most 2^-4 per weight in the normal
  range.  An output element is a weighted mean of V values, so its error is
  at most 2^-4 * max|V| when the weights' errors share one sign; independent
  rounding errors leave about 2^-4 / sqrt(3) ~ 3.6 % of the output's own
  size.  Bar: max |err| <= 2^-4 * max|V| + 2^-7 * max|O|,
  ||err||_2 <= 0.1 * ||O||_2, and mean |err| <= 2^-4 / sqrt(3) * mean |O|:
  with independent zero-mean roundings of relative size at most 2^-4 (the
  kernel divides by the unrounded sum, so err = sum_j p_j eps_j v_j), the
  rms error of an element is at most 2^-4 / sqrt(3) of the rms of the
  weighted values, which on average over many rows is the output's own
  size.  A window one key too wide or too narrow moves a row by about 1/w
  of its weight, far above that.
* Mask edges: closed forms with no weight rounding.  With Q = 0 every
  score is 0 and every weight 2^4 (exact in e4m3), so O is the mean of the
  visible dequantised V rows up to the final bf16 rounding and the fp8
  product's block-sum error (below), and lse = ln(count); with window 1
  each row sees only its own key, so O is that dequantised V row (exact in
  bf16) and lse the diagonal score.
* lse is summed from the unrounded weights, so its error is the scores'
  error.  The fp8 matrix product sums its 64-term blocks with an error of
  up to about 2^-13 of the sum of the terms' magnitudes (measured on this
  instruction), so a score s_ij = sigma q_i . k_j carries up to
  2^-13 |sigma| ||q_i|| ||k_j|| (Cauchy-Schwarz).  Bar per row:
  |err| <= max(1e-3, 2^-12 |sigma| ||q_i|| max_j ||k_j||).
"""

import math
import sys

import numpy as np
import pytest
import torch

from exact_tiled_attention_attn_amd import attn
from exact_tiled_attention_attn_amd.inputs import make_qkv, to_f64
from exact_tiled_attention_attn_amd.workloads import WORKLOADS
from oracle import fp8 as F
from oracle import attention_forward

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    attn.load_library()
    yield
    torch.cuda.synchronize()


def key_of(h, b):
    return 32 * (b // 16) + 8 * ((b % 16) // 4) + 4 * h + b % 4


def expected_vt(codes_v, N):
    """The documented V^T layout built from per-element codes (B, Hkv, N, d)."""
    B, Hkv, _, d = codes_v.shape
    Np = (N + 63) // 64 * 64
    t = np.zeros((B, Hkv, d, Np), dtype=np.uint8)
    t[:, :, :, :N] = np.transpose(codes_v, (0, 1, 3, 2))
    perm = np.array([key_of(p // 32, p % 32) for p in range(64)])
    t = t.reshape(B, Hkv, d, Np // 64, 64)[..., perm].reshape(B, Hkv, d, Np)
    return t


def quantize_gpu(q, k, v):
    q8, k8, vt8, sc = attn.fp8_quantize(q.to(DEV), k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    return q8.cpu().numpy(), k8.cpu().numpy(), vt8.cpu().numpy(), sc.cpu().numpy(), \
        (q8, k8, vt8, sc)


def lse_bound(dq, dk, scale, Hq, Hkv):
    """Per-row lse bound from the dequantised q, k: (B, Hq, N)."""
    qn = np.sqrt((dq * dq).sum(-1))                      # (B, Hq, N)
    kn = np.sqrt((dk * dk).sum(-1)).max(-1)              # (B, Hkv)
    kn = np.repeat(kn, Hq // Hkv, axis=1)[..., None]     # (B, Hq, 1)
    return np.maximum(1e-3, 2.0 ** -12 * abs(scale) * qn * kn)


def check_attention(o, lse, o_ref, l_ref, vmax, lbound, label):
    e = np.abs(to_f64(o) - o_ref)
    el = np.abs(lse.double().numpy() - l_ref)
    fro = np.sqrt((e * e).sum() / (o_ref * o_ref).sum())
    bound = 2.0 ** -4 * vmax + 2.0 ** -7 * np.abs(o_ref).max()
    mean_bound = 2.0 ** -4 / math.sqrt(3.0) * np.abs(o_ref).mean()
    say(f"  {label}: max|err|={e.max():.3e} (bound {bound:.3e}) fro ratio {fro:.3e} "
        f"mean|err|={e.mean():.3e} (bound {mean_bound:.3e}) "
        f"max|dlse|={el.max():.3e} (max ratio to bound {(el / lbound).max():.2f})")
    assert e.max() <= bound and fro <= 0.1 and np.all(el <= lbound), label
    assert e.mean() <= mean_bound, label


SHAPES = [
    # B, Hq, Hkv, N, d, causal, window
    (1, 2, 2, 1, 128, True, 0),
    (1, 2, 2, 65, 64, False, 0),
    (1, 4, 2, 200, 128, True, 0),
    (2, 8, 1, 129, 128, True, 63),
    (1, 16, 2, 1000, 128, True, 0),
    (1, 4, 4, 777, 128, False, 0),
    (1, 6, 2, 300, 128, True, 64),
    (1, 4, 4, 1100, 64, True, 100),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
def test_fp8_codes_and_attention(shape):
    B, Hq, Hkv, N, d, causal, window = shape
    say(f"case fp8 {shape}")
    q, k, v = make_qkv(B, Hq, Hkv, N, d, seed=500 + N + Hq)
    q8, k8, vt8, sc, dev = quantize_gpu(q, k, v)
    o_ref, l_ref, (cq, ck, cv), (sq, sk, sv) = F.fp8_attention_reference(
        to_f64(q), to_f64(k), to_f64(v), 1 / math.sqrt(d), causal, window)
    assert (sc[0], sc[1], sc[2]) == (sq, sk, sv)
    assert np.array_equal(q8, cq) and np.array_equal(k8, ck)
    Np = (N + 63) // 64 * 64
    assert np.array_equal(vt8[:B * Hkv * d * Np].reshape(B, Hkv, d, Np), expected_vt(cv, N))
    o, lse = attn.fwd_fp8(*dev, causal=causal, window=window)
    torch.cuda.synchronize()
    lb = lse_bound(F.e4m3_decode(cq) * sq, F.e4m3_decode(ck) * sk, 1 / math.sqrt(d), Hq, Hkv)
    check_attention(o.cpu(), lse.cpu(), o_ref, l_ref, np.abs(F.e4m3_decode(cv) * sv).max(), lb,
                    str(shape))


@pytest.mark.parametrize("scale", [-0.0883883, 0.5])
def test_fp8_scale_values(scale):
    q, k, v = make_qkv(1, 4, 2, 300, 128, seed=51)
    q = (q.float() * 3.0).to(torch.bfloat16)  # a scale other than the default's
    _, _, _, _, dev = quantize_gpu(q, k, v)
    o_ref, l_ref, (cq, ck, cv), (sq, sk, sv) = F.fp8_attention_reference(
        to_f64(q), to_f64(k), to_f64(v), scale, True, 0)
    o, lse = attn.fwd_fp8(*dev, causal=True, scale=scale)
    torch.cuda.synchronize()
    lb = lse_bound(F.e4m3_decode(cq) * sq, F.e4m3_decode(ck) * sk, scale, 4, 2)
    check_attention(o.cpu(), lse.cpu(), o_ref, l_ref, np.abs(F.e4m3_decode(cv) * sv).max(), lb,
                    f"scale={scale}")


def test_fp8_one_hot_rows_return_the_value_row():
    """Sharp rows: every other weight underflows e4m3 after the 2^8 scaling,
    so O is the retrieved V row up to e4m3 rounding of V itself."""
    N = d = 128
    k = torch.from_numpy(2.0 * np.eye(N, dtype=np.float32))[None, None].to(torch.bfloat16)
    rng = np.random.default_rng(52)
    q = torch.zeros((1, 1, N, d), dtype=torch.bfloat16)
    pick = [int(rng.integers(0, i + 1)) for i in range(N)]
    for i in range(N):
        q[0, 0, i, pick[i]] = 64.0
    v = make_qkv(1, 1, 1, N, d, seed=53)[2]
    _, _, _, _, dev = quantize_gpu(q, k, v)
    o, _ = attn.fwd_fp8(*dev, causal=True, scale=1.0)
    torch.cuda.synchronize()
    _, sv, vdeq = F.quantize(to_f64(v))
    want = vdeq[0, 0, pick]
    np.testing.assert_allclose(to_f64(o.cpu())[0, 0], want, rtol=2 ** -7, atol=1e-6)


EDGE_CASES = [(False, 0), (True, 0), (True, 1), (True, 63), (True, 64), (True, 65), (True, 100)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal,window", EDGE_CASES, ids=[f"c{c}w{w}" for c, w in EDGE_CASES])
def test_fp8_q_zero_is_the_mean_of_the_visible_rows(causal, window, d):
    """Q = 0: O_i is the mean of the dequantised V rows row i sees, which
    are keys max(0, i - w + 1) .. i (causal window), 0 .. i (causal) or all
    (non-causal); lse_i is ln of their number."""
    B, Hq, Hkv, N = 1, 4, 2, 300
    say(f"case fp8 Q=0 causal={causal} window={window} d={d}")
    _, k, v = make_qkv(B, Hq, Hkv, N, d, seed=54 + window)
    q = torch.zeros((B, Hq, N, d), dtype=torch.bfloat16)
    _, _, _, _, dev = quantize_gpu(q, k, v)
    o, lse = attn.fwd_fp8(*dev, causal=causal, window=window, scale=0.125)
    torch.cuda.synchronize()
    o, lse = to_f64(o.cpu()), lse.cpu().double().numpy()
    _, _, vdeq = F.quantize(to_f64(v))
    want = np.zeros((B, Hq, N, d))
    mag = np.zeros((B, Hq, N, d))
    count = np.zeros(N)
    for i in range(N):
        lo = max(0, i - window + 1) if window > 0 else 0
        hi = i + 1 if causal else N
        count[i] = hi - lo
        for h in range(Hq):
            want[0, h, i] = vdeq[0, h // (Hq // Hkv), lo:hi].mean(0)
            mag[0, h, i] = np.abs(vdeq[0, h // (Hq // Hkv), lo:hi]).mean(0)
    err = np.abs(o - want)
    # bf16 rounding of the result, plus the fp8 product's block sums (about
    # 2^-13 of the sum of the terms' magnitudes, taken with a factor 2)
    bound = 2.0 ** -8 * np.abs(want) + 2.0 ** -12 * mag + 1e-6
    say(f"  max|err| {err.max():.3e}, max ratio to bound {(err / bound).max():.3f}, "
        f"max|dlse| {np.abs(lse - np.log(count)).max():.3e}")
    assert np.all(err <= bound)
    assert np.all(np.abs(lse - np.log(count)[None, None]) <= 1e-5)


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_window_one_returns_the_own_value_row(d):
    B, Hq, Hkv, N = 2, 4, 1, 200
    say(f"case fp8 window=1 d={d}")
    q, k, v = make_qkv(B, Hq, Hkv, N, d, seed=55)
    _, _, _, _, dev = quantize_gpu(q, k, v)
    sigma = 1 / math.sqrt(d)
    o, lse = attn.fwd_fp8(*dev, causal=True, window=1, scale=sigma)
    torch.cuda.synchronize()
    _, _, dq = F.quantize(to_f64(q))
    _, _, dk = F.quantize(to_f64(k))
    _, _, dv = F.quantize(to_f64(v))
    G = Hq // Hkv
    own_v = np.repeat(dv, G, axis=1)
    assert np.array_equal(to_f64(o.cpu()), own_v)
    diag = float(np.float32(sigma)) * (dq * np.repeat(dk, G, axis=1)).sum(-1)
    el = np.abs(lse.cpu().double().numpy() - diag)
    lb = lse_bound(dq, dk, sigma, Hq, Hkv)
    say(f"  max|dlse| {el.max():.3e} (max ratio to bound {(el / lb).max():.2f})")
    assert np.all(el <= lb)


@pytest.mark.parametrize("name", ["c2_causal_mha", "c4_causal_gqa"])
def test_fp8_workload_every_row(name):
    w = WORKLOADS[name]
    say(f"case fp8 workload {name}")
    q, k, v = make_qkv(w.B, w.Hq, w.Hkv, w.N, w.d, w.seed)
    q8, k8, vt8, sc, dev = quantize_gpu(q, k, v)
    o, lse = attn.fwd_fp8(*dev, causal=w.causal, window=w.window, scale=w.sm_scale)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    say("  HIP done; oracle")
    from threadpoolctl import threadpool_limits
    cq, sq, dq = F.quantize(q.float().numpy())
    ck, sk, dk = F.quantize(k.float().numpy())
    cv, sv, dv = F.quantize(v.float().numpy())
    assert (sc[0], sc[1], sc[2]) == (sq, sk, sv)
    assert np.array_equal(q8, cq) and np.array_equal(k8, ck)
    with threadpool_limits(limits=1, user_api="blas"):
        o_ref, l_ref = attention_forward(dq, dk, dv, w.sm_scale, w.causal, w.window, workers=16)
    check_attention(o, lse, o_ref, l_ref, np.abs(dv).max(),
                    lse_bound(dq, dk, w.sm_scale, w.Hq, w.Hkv), name)
