"""GPU parity of the packed-sequence forward with structured masks
(attn_fwd_varlen) against the float64 oracle.

Bar (the forward's): O max |err| <= 2e-2, mean |err| <= 2e-3, lse max |err|
<= 1e-3, on every row of every head, including the full-size packed and
Longformer workloads.
"""

import math
import sys

import numpy as np
import pytest
import torch

from exact_tiled_attention_attn_amd import attn
from exact_tiled_attention_attn_amd.inputs import make_packed_qkv, make_qkv, to_f64
from exact_tiled_attention_attn_amd.workloads import VARLEN_WORKLOADS
from oracle import attention_general

pytestmark = pytest.mark.gpu

O_MAX, O_MEAN, LSE_MAX = 2e-2, 2e-3, 1e-3
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


def run(q, k, v, cu, causal, window=0, radius=0, n_global=0, scale=None, max_len=None):
    lens = (cu[1:] - cu[:-1]).tolist()
    o, lse = attn.fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV),
                             max_len if max_len is not None else max(lens), causal=causal,
                             window=window, radius=radius, n_global=n_global, scale=scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def check(o, lse, o_ref, l_ref, label):
    eo = np.abs(to_f64(o) - o_ref)
    el = np.abs(lse.double().numpy() - l_ref)
    say(f"  {label}: max|dO|={eo.max():.3e} mean|dO|={eo.mean():.3e} max|dlse|={el.max():.3e}")
    assert np.isfinite(eo.max()) and np.isfinite(el.max()), label
    assert eo.max() <= O_MAX and eo.mean() <= O_MEAN and el.max() <= LSE_MAX, label


CASES = [
    # lens, Hq, Hkv, d, causal, window, radius, n_global
    ([1], 2, 2, 128, False, 0, 0, 0),
    ([63, 64, 65, 1, 200], 4, 2, 128, False, 0, 0, 0),
    ([63, 64, 65, 1, 200], 4, 2, 128, True, 0, 0, 0),
    ([300, 7, 513], 8, 1, 128, True, 50, 0, 0),
    ([1000, 129], 4, 4, 64, False, 0, 100, 0),          # band only
    ([1000, 129, 700], 4, 4, 64, False, 0, 100, 5),     # band + global tokens
    ([1000, 64], 4, 2, 128, True, 0, 70, 40),           # causal band + globals
    ([900], 2, 2, 128, True, 200, 0, 100),              # causal window + globals
    ([777, 33], 8, 2, 128, False, 0, 0, 64),            # globals, no band: full rows
    ([2048, 5, 1500], 16, 2, 128, False, 0, 256, 16),   # Longformer-like
    ([4096], 4, 4, 64, False, 0, 256, 300),             # more globals than a tile
    ([31, 32, 33, 100, 1], 4, 4, 64, True, 0, 8, 33),   # two global blocks, short sequences
    ([3000, 40], 8, 4, 128, False, 0, 128, 20),         # d = 128 Longformer-like
    # more than 64 sequences of different lengths: the compacted launch
    # order scans the lengths in chunks of 64 per wave
    ([int(x) for x in np.random.default_rng(7).integers(0, 300, size=150)],
     4, 2, 64, True, 0, 0, 0),
    ([int(x) for x in np.random.default_rng(8).integers(1, 200, size=70)],
     8, 8, 128, False, 0, 30, 2),
]


def case_id(c):
    lens = c[0]
    short = str(lens) if len(lens) <= 8 else f"[{len(lens)} lengths, total {sum(lens)}]"
    return str((short,) + tuple(c[1:]))


@pytest.mark.parametrize("case", CASES, ids=[case_id(c) for c in CASES])
def test_varlen_parity(case):
    lens, Hq, Hkv, d, causal, window, radius, n_global = case
    say(f"case varlen {case_id(case)}")
    q, k, v, cu = make_packed_qkv(lens, Hq, Hkv, d, seed=300 + len(lens) + Hq)
    o, lse = run(q, k, v, cu, causal, window, radius, n_global)
    o_ref, l_ref = attention_general(to_f64(q), to_f64(k), to_f64(v), 1 / math.sqrt(d),
                                     cu.tolist(), causal, window, radius, n_global)
    check(o, lse, o_ref, l_ref, str(case))


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 100)])
def test_one_sequence_equals_the_dense_forward_bitwise(causal, window):
    """Without band or globals, one packed sequence is the dense problem and
    goes through the same tiles in the same order."""
    q, k, v = make_qkv(1, 8, 2, 1000, 128, seed=41)
    cu = torch.tensor([0, 1000], dtype=torch.int32)
    ov, lv = run(q[0], k[0], v[0], cu, causal, window)
    od, ld = attn.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, window=window)
    assert torch.equal(ov, od.cpu()[0]) and torch.equal(lv, ld.cpu()[0])


def test_larger_max_seqlen_and_empty_sequences():
    """A max_seqlen above the longest sequence only adds workgroups that exit;
    zero-length sequences are allowed."""
    lens = [0, 100, 0, 250]
    q, k, v, cu = make_packed_qkv(lens, 4, 2, 128, seed=42)
    o1, l1 = run(q, k, v, cu, True, 0, 0, 3)
    o2, l2 = run(q, k, v, cu, True, 0, 0, 3, max_len=5000)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o_ref, l_ref = attention_general(to_f64(q), to_f64(k), to_f64(v), 1 / math.sqrt(128),
                                     cu.tolist(), True, 0, 0, 3)
    check(o1, l1, o_ref, l_ref, "empty sequences")


@pytest.mark.parametrize("name", list(VARLEN_WORKLOADS))
def test_varlen_workload_parity(name):
    w = VARLEN_WORKLOADS[name]
    say(f"case varlen workload {name} total={w.total}")
    q, k, v, cu = make_packed_qkv(list(w.lens), w.Hq, w.Hkv, w.d, seed=w.seed)
    o, lse = run(q, k, v, cu, w.causal, w.window, w.radius, w.n_global, scale=w.sm_scale)
    say("  HIP done; oracle")
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1, user_api="blas"):
        o_ref, l_ref = attention_general(q.float().numpy(), k.float().numpy(),
                                         v.float().numpy(), w.sm_scale, cu.tolist(), w.causal,
                                         w.window, w.radius, w.n_global, block=256, workers=16)
    check(o, lse, o_ref, l_ref, name)
