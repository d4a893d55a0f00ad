"""GPU parity of the backward (dQ, dK, dV) against the float64 gradient oracle.

The HIP forward supplies o and lse, as in training; the HIP backward then
runs through the C ABI.  The oracle computes the exact gradients of the same
bf16 inputs in float64.

Bar, for each of dQ, dK and dV (errors against the unrounded oracle, n
elements):
    max |err|   <= 1e-2 * max |ref|   + 1e-5
    ||err||_2   <= 1e-2 * ||ref||_2   + 1e-5 * sqrt(n)
Every output element is a sum of products whose one rounded operand (P for
dV, dS for dQ and dK, rounded to bf16 for the matrix cores) carries at most
2^-9 relative error, plus the final rounding to bf16 (2^-9); with the
rounding errors of independent terms adding like a random walk, the relative
Frobenius error is about 2^-9 (2e-3), and a plausible mistake (a dropped
Delta, a wrong scale, a missing mask, a transposed operand) moves it to
order one.  The absolute floor covers gradients that are exactly zero in the
exact result (a row that sees one key has dS = 0), where fp32 summation in a
different order than Delta's leaves about 1e-7.
"""

import math
import sys

import numpy as np
import pytest
import torch

from exact_tiled_attention_attn_amd import attn
from exact_tiled_attention_attn_amd.inputs import make_dout, make_qkv, to_f64
from exact_tiled_attention_attn_amd.workloads import WORKLOADS
from oracle import attention_backward

pytestmark = pytest.mark.gpu

REL_MAX, REL_FRO, ABS_FLOOR = 1e-2, 1e-2, 1e-5
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


def run(q, k, v, do, causal, window, scale=None):
    """CPU bf16 in; HIP forward then HIP backward; CPU bf16 (dq, dk, dv) out."""
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, lse = attn.fwd(qd, kd, vd, causal=causal, window=window, scale=scale)
    dq, dk, dv = attn.bwd(qd, kd, vd, o, lse, dod, causal=causal, window=window, scale=scale)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def check(got, ref, label):
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        e = np.abs(to_f64(g) - r)
        emax, rmax = e.max(), np.abs(r).max()
        efro, rfro = np.sqrt((e * e).sum()), np.sqrt((r * r).sum())
        say(f"  {label} {name}: max|err|={emax:.3e} (ref {rmax:.3e}, ratio {emax / max(rmax, 1e-30):.2e})"
            f" fro ratio {efro / max(rfro, 1e-30):.2e}")
        assert np.isfinite(emax), f"{label} {name}"
        assert emax <= REL_MAX * rmax + ABS_FLOOR, f"{label} {name}: max|err| {emax} vs {rmax}"
        assert efro <= REL_FRO * rfro + ABS_FLOOR * math.sqrt(e.size), \
            f"{label} {name}: fro {efro} vs {rfro}"


def oracle(q, k, v, do, scale, causal, window, workers=1):
    return attention_backward(to_f64(q), to_f64(k), to_f64(v), to_f64(do), scale, causal, window,
                              workers=workers)


SHAPES = [
    # B, Hq, Hkv, N, d, causal, window
    (1, 2, 2, 1, 128, True, 0),
    (1, 2, 2, 7, 64, False, 0),
    (1, 2, 1, 63, 128, True, 0),
    (1, 4, 4, 64, 128, True, 0),
    (1, 4, 2, 65, 128, True, 2),
    (2, 8, 1, 129, 128, True, 63),     # multi-query
    (1, 4, 4, 200, 128, False, 0),
    (1, 8, 8, 1000, 128, True, 65),
    (1, 16, 2, 1000, 128, True, 0),    # group of 8
    (1, 6, 2, 300, 128, True, 64),     # group of 3
    (1, 12, 6, 640, 128, True, 200),   # group of 2
    (1, 4, 2, 777, 64, False, 0),
    (1, 4, 4, 513, 128, False, 0),
    (2, 4, 4, 257, 128, True, 1),
    (1, 2, 2, 300, 128, True, 4096),   # window >= N
    (1, 4, 4, 1100, 64, True, 100),
    (1, 2, 2, 1029, 64, True, 0),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
def test_bwd_parity_small_shapes(shape):
    B, Hq, Hkv, N, d, causal, window = shape
    say(f"case bwd {shape}")
    q, k, v = make_qkv(B, Hq, Hkv, N, d, seed=2000 + N + Hq)
    do = make_dout(B, Hq, N, d, seed=3000 + N)
    got = run(q, k, v, do, causal, window)
    ref = oracle(q, k, v, do, 1 / math.sqrt(d), causal, window)
    check(got, ref, str(shape))


@pytest.mark.parametrize("scale", [-0.0883883, 0.5, 1e-6])
def test_bwd_scale_values(scale):
    q, k, v = make_qkv(1, 4, 2, 300, 128, seed=21)
    do = make_dout(1, 4, 300, 128, seed=22)
    say(f"case bwd scale={scale}")
    got = run(q, k, v, do, True, 0, scale=scale)
    ref = oracle(q, k, v, do, scale, True, 0)
    check(got, ref, f"scale={scale}")


def test_bwd_zero_scale():
    """scale = 0: uniform weights, so dQ = dK = 0 exactly and dV_j is the sum
    of dO_i / |V_i| over the rows that see j."""
    q, k, v = make_qkv(1, 2, 2, 300, 128, seed=23)
    do = make_dout(1, 2, 300, 128, seed=24)
    say("case bwd scale=0")
    dq, dk, dv = run(q, k, v, do, True, 0, scale=0.0)
    assert not dq.float().abs().max() and not dk.float().abs().max()
    ref = oracle(q, k, v, do, 0.0, True, 0)
    check((dq, dk, dv), ref, "scale=0")


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 37)])
def test_bwd_zero_query_closed_form(causal, window):
    """Q = 0: row i weights its |V_i| visible keys equally, so
    dV_j = sum over the rows i that see j of dO_i / |V_i| (no oracle)."""
    N, d = 500, 128
    _, k, v = make_qkv(1, 1, 1, N, d, seed=25)
    q = torch.zeros((1, 1, N, d), dtype=torch.bfloat16)
    do = make_dout(1, 1, N, d, seed=26)
    say(f"case bwd Q=0 {causal} {window}")
    _, _, dv = run(q, k, v, do, causal, window)
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    vis = np.ones((N, N), dtype=bool)
    if causal:
        vis &= j <= i
    if window:
        vis &= j > i - window
    p = vis / vis.sum(1, keepdims=True)
    want = p.T @ to_f64(do)[0, 0]
    got = to_f64(dv)[0, 0]
    e = np.abs(got - want)
    assert e.max() <= REL_MAX * np.abs(want).max()
    assert np.sqrt((e * e).sum()) <= REL_FRO * np.sqrt((want * want).sum())


def test_bwd_window_one_passes_dout_through():
    """w = 1: each row sees only itself with weight 1, so dV = dO (summed over
    the group) and dQ = dK = 0 up to summation order."""
    N, d, Hq, Hkv = 333, 128, 4, 2
    q, k, v = make_qkv(1, Hq, Hkv, N, d, seed=27)
    do = make_dout(1, Hq, N, d, seed=28)
    say("case bwd window=1")
    dq, dk, dv = run(q, k, v, do, True, 1)
    want = do.float().view(1, Hkv, Hq // Hkv, N, d).sum(2)
    assert (dv.float() - want).abs().max() <= 2 ** -8 * want.abs().max()
    assert dq.float().abs().max() <= 1e-3 and dk.float().abs().max() <= 1e-3


def test_bwd_constant_v_has_no_query_or_key_gradient():
    q, k, _ = make_qkv(1, 2, 2, 400, 128, seed=29)
    v = torch.full((1, 2, 400, 128), -1.375, dtype=torch.bfloat16)
    do = make_dout(1, 2, 400, 128, seed=30)
    say("case bwd constant V")
    dq, dk, dv = run(q, k, v, do, True, 0)
    ref = oracle(q, k, v, do, 1 / math.sqrt(128), True, 0)
    scale = np.abs(ref[2]).max()
    assert dq.float().abs().max() <= 1e-2 * scale and dk.float().abs().max() <= 1e-2 * scale
    check((torch.zeros_like(dq), torch.zeros_like(dk), dv), (ref[0] * 0, ref[1] * 0, ref[2]),
          "constant V (dv)")


def test_bwd_gqa_equals_repeated_mha_summed():
    N, d, Hq, Hkv = 600, 128, 16, 2
    G = Hq // Hkv
    q, k, v = make_qkv(1, Hq, Hkv, N, d, seed=31)
    do = make_dout(1, Hq, N, d, seed=32)
    say("case bwd GQA vs repeated MHA")
    gq, gk, gv = run(q, k, v, do, True, 0)
    mq, mk, mv = run(q, k.repeat_interleave(G, dim=1).contiguous(),
                     v.repeat_interleave(G, dim=1).contiguous(), do, True, 0)
    assert (gq.float() - mq.float()).abs().max() <= 1e-2 * mq.float().abs().max()
    for g, m in ((gk, mk), (gv, mv)):
        summed = m.float().view(1, Hkv, G, N, d).sum(2)
        assert (g.float() - summed).abs().max() <= 2e-2 * summed.abs().max()


def test_bwd_deterministic_and_guard_bands():
    B, Hq, Hkv, N, d = 1, 4, 2, 333, 128
    q, k, v = (t.to(DEV) for t in make_qkv(B, Hq, Hkv, N, d, seed=33))
    do = make_dout(B, Hq, N, d, seed=34).to(DEV)
    o, lse = attn.fwd(q, k, v, causal=True, window=100)
    pad = 4096
    say("case bwd guard bands")
    results = []
    for _ in range(2):
        bufs, views = [], []
        for H in (Hq, Hkv, Hkv):
            buf = torch.full((H * N * d + 2 * pad,), 7.0, dtype=torch.bfloat16, device=DEV)
            bufs.append((buf, H * N * d))
            views.append(buf[pad:pad + H * N * d].view(B, H, N, d))
        nws = attn.attn_bwd_workspace_size(B, Hq, N) // 4
        ws = torch.full((nws + 2 * pad,), 7.0, dtype=torch.float32, device=DEV)
        attn.bwd(q, k, v, o, lse, do, causal=True, window=100, out=tuple(views),
                 workspace=ws[pad:pad + nws])
        torch.cuda.synchronize()
        for buf, n in bufs + [(ws, nws)]:
            assert bool((buf[:pad] == 7.0).all()) and bool((buf[pad + n:] == 7.0).all())
        results.append([t.clone() for t in views])
    for a, b in zip(*results):
        assert torch.equal(a, b)


def test_bwd_empty_problems_and_side_stream():
    e = torch.empty((0, 2, 16, 128), dtype=torch.bfloat16, device=DEV)
    el = torch.empty((0, 2, 16), dtype=torch.float32, device=DEV)
    dq, dk, dv = attn.bwd(e, e, e, e, el, e, causal=True)
    assert dq.shape == e.shape
    q, k, v = make_qkv(1, 2, 2, 200, 128, seed=35)
    do = make_dout(1, 2, 200, 128, seed=36)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
        o, lse = attn.fwd(qd, kd, vd, causal=True)
        got = attn.bwd(qd, kd, vd, o, lse, dod, causal=True)
    s.synchronize()
    check([t.cpu() for t in got], oracle(q, k, v, do, 1 / math.sqrt(128), True, 0), "side stream")


# ---------------------------------------------------------------------------
# full-size workloads, every element: the oracle covers them in tens of
# seconds on the host cores
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["c2_causal_mha", "c2_causal_mha_sharp", "c3_causal_window",
                                  "c4_causal_gqa"])
def test_bwd_workload_parity(name):
    w = WORKLOADS[name]
    say(f"case bwd workload {name}")
    q, k, v = make_qkv(w.B, w.Hq, w.Hkv, w.N, w.d, w.seed)
    if w.q_mult != 1.0:
        q = (q.float() * w.q_mult).to(torch.bfloat16)  # exact: power of two
    do = make_dout(w.B, w.Hq, w.N, w.d, w.seed + 100)
    got = run(q, k, v, do, w.causal, w.window, scale=w.sm_scale)
    say("  HIP done; oracle")
    from threadpoolctl import threadpool_limits
    qf, kf, vf, dof = (t.float().numpy() for t in (q, k, v, do))
    with threadpool_limits(limits=1, user_api="blas"):
        ref = attention_backward(qf, kf, vf, dof, w.sm_scale, w.causal, w.window, workers=16)
    check(got, ref, name)
