"""The allocation-free paged decode (attn_decode_paged_noalloc) against the
decode entry point that takes a workspace, through the C ABI: the same
kernels and key split, so the outputs must be bitwise equal.  Two calls in a
row, the second smaller (the scratch keeps the first call's partials), then
the first size again; and the oracle bar on the first case."""

import math
import sys

import numpy as np
import pytest
import torch

from exact_tiled_attention_attn_amd import attn
from exact_tiled_attention_attn_amd.inputs import decode_lengths, make_decode_q, make_paged_kv, to_f64
from oracle import decode_paged

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


def _problem(B, Hq, Hkv, T, d, page_size, max_len, seed, window=0):
    lens = decode_lengths(B, max_len, seed)
    kc, vc, table = make_paged_kv(lens, Hkv, d, page_size, seed=seed)
    q = make_decode_q(B, Hq, T, d, seed=seed + 1)
    return dict(q=q.to(DEV), kc=kc.to(DEV), vc=vc.to(DEV), table=table.to(DEV),
                lens=torch.tensor(lens, dtype=torch.int32, device=DEV), lens_list=lens, B=B,
                Hq=Hq, Hkv=Hkv, T=T, d=d, page_size=page_size, max_len=max_len, window=window,
                host=(q, kc, vc, table))


def _both(p):
    scale = 1.0 / math.sqrt(p["d"])
    args = (p["B"], p["Hq"], p["Hkv"], p["T"], p["d"], p["page_size"], p["kc"].shape[0],
            p["table"].shape[1], p["max_len"], scale, p["window"])
    o1 = torch.empty_like(p["q"])
    l1 = torch.empty((p["B"], p["Hq"], p["T"]), dtype=torch.float32, device=DEV)
    nbytes = attn.attn_decode_workspace_size(p["B"], p["Hq"], p["Hkv"], p["T"], p["d"],
                                             p["page_size"], p["max_len"], p["window"])
    ws = torch.empty((max(nbytes, 16) // 4,), dtype=torch.float32, device=DEV)
    st = attn.attn_decode_paged(p["q"], p["kc"], p["vc"], p["table"], p["lens"], o1, l1, ws, *args)
    assert st == attn.ATTN_OK, attn.attn_status_string(st)
    o2 = torch.full_like(p["q"], 7.0)
    l2 = torch.full((p["B"], p["Hq"], p["T"]), 7.0, dtype=torch.float32, device=DEV)
    st = attn.attn_decode_paged_noalloc(p["q"], p["kc"], p["vc"], p["table"], p["lens"], o2, l2,
                                        *args)
    assert st == attn.ATTN_OK, attn.attn_status_string(st)
    torch.cuda.synchronize()
    return (o1.cpu(), l1.cpu()), (o2.cpu(), l2.cpu())


def test_noalloc_matches_the_workspace_entry_point_with_many_columns():
    """More than 32 query columns per KV head (the multi-wave kernel):
    multi-query at 64 heads, then 16 heads x 4 tokens with a window."""
    for label, p in (("multi-query 64/1", _problem(4, 64, 1, 1, 128, 64, 40000, seed=31)),
                     ("16 heads x 4 tokens, window", _problem(2, 32, 2, 4, 64, 16, 9000, seed=32,
                                                             window=2000))):
        say(f"case noalloc {label}")
        (o1, l1), (o2, l2) = _both(p)
        assert torch.equal(o1, o2), label
        assert torch.equal(l1, l2), label


def test_noalloc_matches_the_workspace_entry_point_on_two_calls_in_a_row():
    big = _problem(8, 64, 8, 1, 128, 64, 131072, seed=21)
    small = _problem(3, 16, 2, 4, 128, 32, 3000, seed=7, window=700)
    for label, p in (("128k GQA decode", big), ("small windowed, 4 tokens", small),
                     ("128k GQA decode again", big)):
        say(f"case noalloc {label}")
        (o1, l1), (o2, l2) = _both(p)
        assert torch.equal(o1, o2), label
        assert torch.equal(l1, l2), label
    # and the bar against the oracle on the small case
    q, kc, vc, table = small["host"]
    o_ref, l_ref = decode_paged(to_f64(q), to_f64(kc), to_f64(vc), table.numpy(),
                                small["lens_list"], 1.0 / math.sqrt(128), small["window"])
    (_, _), (o2, l2) = _both(small)
    fin = np.isfinite(l_ref)
    eo = np.abs(to_f64(o2) - o_ref)[fin]
    el = np.abs(l2.double().numpy() - l_ref)[fin]
    say(f"  small vs oracle: max|dO|={eo.max():.3e} mean|dO|={eo.mean():.3e} "
        f"max|dlse|={el.max():.3e}")
    assert eo.max() <= 2e-2 and eo.mean() <= 2e-3 and el.max() <= 1e-3


def test_noalloc_rejects_a_problem_beyond_the_scratch():
    q = torch.empty((8, 256, 1, 128), dtype=torch.bfloat16, device=DEV)
    o = torch.empty_like(q)
    lse = torch.empty((8, 256, 1), dtype=torch.float32, device=DEV)
    kc = torch.empty((16, 64, 8, 128), dtype=torch.bfloat16, device=DEV)
    table = torch.zeros((8, 2048), dtype=torch.int32, device=DEV)
    lens = torch.zeros((8,), dtype=torch.int32, device=DEV)
    st = attn.attn_decode_paged_noalloc(q, kc, kc, table, lens, o, lse, 8, 256, 8, 1, 128, 64, 16,
                                        2048, 131072, 0.1, 0)
    assert st == attn.ATTN_ERR_NO_SCRATCH
