"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before any HIP call (so these
calls launch nothing and never touch the fake pointers passed in)."""

import os
import re

import pytest

from exact_tiled_attention_attn_amd import attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

# fake, 16-byte aligned, never dereferenced: every call below fails validation
P = 0x10000


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(attn.LIB_PATH):
        from exact_tiled_attention_attn_amd.build import build
        build(verbose=False)
    return attn.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))


def test_header_declares_the_expected_entry_points():
    assert _declared_functions() == sorted(attn.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_constants_match_header(lib):
    text = open(HEADER).read()
    assert int(re.search(r"#define ATTN_ABI_VERSION (\d+)", text).group(1)) == lib.attn_abi_version()
    assert "(1 << 22)" in text and attn.ATTN_MAX_N == 1 << 22
    for name, val in (("ATTN_OK", 0), ("ATTN_ERR_INVALID_ARG", 1), ("ATTN_ERR_UNSUPPORTED", 2),
                      ("ATTN_ERR_LAUNCH", 3), ("ATTN_ERR_NO_SCRATCH", 4)):
        assert re.search(rf"{name} = {val}\b", text)
        assert getattr(attn, name) == val


def test_device_info_rejects_a_negative_device(lib):
    import ctypes
    x = ctypes.c_int(-5)
    assert lib.attn_device_info(-1, ctypes.byref(x), None, None, None) == attn.ATTN_ERR_INVALID_ARG
    assert x.value == -5
    with pytest.raises(attn.AttnError):
        attn.attn_device_info(-1)


def test_status_strings_and_variants(lib):
    assert attn.attn_status_string(0) == "ok"
    assert attn.attn_status_string(1) == "invalid argument"
    assert attn.attn_status_string(2) == "unsupported problem"
    assert attn.attn_status_string(3) == "kernel launch failed"
    assert attn.attn_status_string(4) == "problem exceeds the allocation-free scratch"
    assert attn.attn_status_string(99) == "unknown status"
    n = attn.attn_num_variants()
    assert n >= 2
    assert attn.attn_variant_name(0) == "auto"
    names = [attn.attn_variant_name(i) for i in range(n)]
    assert len(set(names)) == n and "invalid" not in names
    assert attn.attn_variant_name(n) == "invalid"
    assert attn.attn_variant_name(-1) == "invalid"


GOOD = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=4, Hkv=2, N=64, d=128, scale=0.1, causal=1,
            window=0)


def call(**kw):
    a = dict(GOOD)
    a.update(kw)
    variant = a.pop("variant", None)
    if variant is None:
        return attn.attn_fwd(**a)
    return attn.attn_fwd_ex(**a, variant=variant)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(k=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(v=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(o=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(lse=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(B=-1), attn.ATTN_ERR_INVALID_ARG),
    (dict(N=-5), attn.ATTN_ERR_INVALID_ARG),
    (dict(Hq=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(Hkv=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(Hq=6, Hkv=4), attn.ATTN_ERR_INVALID_ARG),     # Hq % Hkv != 0
    (dict(causal=2), attn.ATTN_ERR_INVALID_ARG),
    (dict(scale=float("nan")), attn.ATTN_ERR_INVALID_ARG),
    (dict(scale=float("inf")), attn.ATTN_ERR_INVALID_ARG),
    (dict(variant=-1), attn.ATTN_ERR_INVALID_ARG),
    (dict(variant=99), attn.ATTN_ERR_INVALID_ARG),
    (dict(d=96), attn.ATTN_ERR_UNSUPPORTED),
    (dict(d=256), attn.ATTN_ERR_UNSUPPORTED),
    (dict(causal=0, window=16), attn.ATTN_ERR_UNSUPPORTED),  # window needs causal
    (dict(q=P + 8), attn.ATTN_ERR_UNSUPPORTED),               # misaligned
    (dict(lse=P + 4), attn.ATTN_ERR_UNSUPPORTED),
    (dict(N=(1 << 22) + 1), attn.ATTN_ERR_UNSUPPORTED),
])
def test_rejects_bad_arguments_without_launching(lib, kw, expect):
    assert call(**kw) == expect


@pytest.mark.parametrize("kw", [dict(B=0), dict(N=0), dict(B=0, q=0, k=0, v=0, o=0, lse=0),
                                dict(N=0, q=0, k=0, v=0, o=0, lse=0)])
def test_empty_problem_is_ok_and_launches_nothing(lib, kw):
    # nothing is launched, so this is safe without a GPU and with null pointers
    assert call(**kw) == attn.ATTN_OK


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(attn, "_lib", None)
    monkeypatch.setattr(attn, "LIB_PATH", str(tmp_path / "libattn.so"))
    with pytest.raises(attn.AttnError):
        attn.load_library()


def test_fwd_wrapper_rejects_host_tensors(lib):
    import torch
    q = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16)
    with pytest.raises(attn.AttnError):
        attn.fwd(q, q, q)


def test_caller_buffers_are_checked_before_the_call():
    """out= buffers and workspaces the caller passes are checked in the
    binding (the C entry points cannot see their extent); the same helpers
    run in fwd, fwd_varlen, fwd_fp8, bwd and decode before the call."""
    import torch
    dev = torch.device("cpu")
    good = torch.empty((2, 3, 4), dtype=torch.bfloat16)
    attn._check_out(good, (2, 3, 4), torch.bfloat16, dev, "o")
    for bad in (torch.empty((2, 3, 5), dtype=torch.bfloat16),
                torch.empty((2, 3, 4), dtype=torch.float32),
                torch.empty((2, 4, 3), dtype=torch.bfloat16).transpose(1, 2)):
        with pytest.raises(attn.AttnError):
            attn._check_out(bad, (2, 3, 4), torch.bfloat16, dev, "o")
    with pytest.raises(attn.AttnError):
        attn._check_out(good, (2, 3, 4), torch.bfloat16, torch.device("meta"), "o")
    ws = torch.empty((100,), dtype=torch.float32)
    attn._check_workspace(ws, 400, dev)
    with pytest.raises(attn.AttnError):
        attn._check_workspace(ws, 401, dev)
    with pytest.raises(attn.AttnError):
        attn._check_workspace(torch.empty((10, 20), dtype=torch.float32).t(), 4, dev)


BWD_GOOD = dict(q=P, k=P, v=P, o=P, lse=P, dout=P, dq=P, dk=P, dv=P, workspace=P, B=1, Hq=4,
                Hkv=2, N=64, d=128, scale=0.1, causal=1, window=0)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(o=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(lse=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(dout=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(dq=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(dk=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(dv=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(workspace=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(B=-1), attn.ATTN_ERR_INVALID_ARG),
    (dict(Hq=6, Hkv=4), attn.ATTN_ERR_INVALID_ARG),
    (dict(causal=3), attn.ATTN_ERR_INVALID_ARG),
    (dict(scale=float("nan")), attn.ATTN_ERR_INVALID_ARG),
    (dict(d=32), attn.ATTN_ERR_UNSUPPORTED),
    (dict(causal=0, window=8), attn.ATTN_ERR_UNSUPPORTED),
    (dict(dv=P + 2), attn.ATTN_ERR_UNSUPPORTED),
    (dict(workspace=P + 4), attn.ATTN_ERR_UNSUPPORTED),
    (dict(N=(1 << 22) + 1), attn.ATTN_ERR_UNSUPPORTED),
])
def test_bwd_rejects_bad_arguments_without_launching(lib, kw, expect):
    a = dict(BWD_GOOD)
    a.update(kw)
    assert attn.attn_bwd(**a) == expect


@pytest.mark.parametrize("kw", [dict(B=0), dict(N=0),
                                dict(N=0, q=0, k=0, v=0, o=0, lse=0, dout=0, dq=0, dk=0, dv=0,
                                     workspace=0)])
def test_bwd_empty_problem_is_ok_and_launches_nothing(lib, kw):
    a = dict(BWD_GOOD)
    a.update(kw)
    assert attn.attn_bwd(**a) == attn.ATTN_OK


def test_bwd_workspace_size(lib):
    assert attn.attn_bwd_workspace_size(2, 32, 8192) == 2 * 32 * 8192 * 4
    assert attn.attn_bwd_workspace_size(0, 32, 8192) == 0
    assert attn.attn_bwd_workspace_size(1, 1, -3) == 0
    assert attn.attn_bwd_workspace_size(3, 64, 1 << 22) == 3 * 64 * (1 << 22) * 4


DEC_GOOD = dict(q=P, k_cache=P, v_cache=P, block_table=P, seq_lens=P, o=P, lse=P, workspace=P,
                B=2, Hq=8, Hkv=2, T=1, d=128, page_size=16, num_pages=10,
                max_pages_per_seq=5, max_seq_len=80, scale=0.1, window=0)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(k_cache=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(block_table=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(seq_lens=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(workspace=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(lse=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(B=-1), attn.ATTN_ERR_INVALID_ARG),
    (dict(T=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(Hq=6, Hkv=4), attn.ATTN_ERR_INVALID_ARG),
    (dict(num_pages=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(max_pages_per_seq=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(scale=float("nan")), attn.ATTN_ERR_INVALID_ARG),
    (dict(d=96), attn.ATTN_ERR_UNSUPPORTED),
    (dict(page_size=24), attn.ATTN_ERR_UNSUPPORTED),     # not a power of two
    (dict(page_size=8), attn.ATTN_ERR_UNSUPPORTED),
    (dict(page_size=8192), attn.ATTN_ERR_UNSUPPORTED),
    (dict(T=257), attn.ATTN_ERR_UNSUPPORTED),            # 4 heads x 257 tokens > 1024
    (dict(block_table=P + 2), attn.ATTN_ERR_UNSUPPORTED),
    (dict(o=P + 8), attn.ATTN_ERR_UNSUPPORTED),
    (dict(max_seq_len=(1 << 22) + 1), attn.ATTN_ERR_UNSUPPORTED),
])
def test_decode_rejects_bad_arguments_without_launching(lib, kw, expect):
    a = dict(DEC_GOOD)
    a.update(kw)
    assert attn.attn_decode_paged(**a) == expect


@pytest.mark.parametrize("kw", [dict(B=0), dict(max_seq_len=0),
                                dict(B=0, q=0, k_cache=0, v_cache=0, block_table=0, seq_lens=0,
                                     o=0, lse=0, workspace=0)])
def test_decode_empty_problem_is_ok_and_launches_nothing(lib, kw):
    a = dict(DEC_GOOD)
    a.update(kw)
    assert attn.attn_decode_paged(**a) == attn.ATTN_OK


NOALLOC_GOOD = {k: v for k, v in DEC_GOOD.items() if k != "workspace"}


@pytest.mark.parametrize("kw,expect", [
    (dict(q=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(lse=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(T=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(d=96), attn.ATTN_ERR_UNSUPPORTED),
    (dict(T=257), attn.ATTN_ERR_UNSUPPORTED),
    (dict(o=P + 8), attn.ATTN_ERR_UNSUPPORTED),
    # 64 sequences x 8 KV heads x 32 columns of a 128k cache: 67.6 MB of
    # partials, more than the 32 MiB scratch
    (dict(B=8, Hq=256, Hkv=8, T=1, page_size=64, max_pages_per_seq=2048, num_pages=16384,
          max_seq_len=131072), attn.ATTN_ERR_NO_SCRATCH),
])
def test_decode_noalloc_rejects_without_launching(lib, kw, expect):
    a = dict(NOALLOC_GOOD)
    a.update(kw)
    assert attn.attn_decode_paged_noalloc(**a) == expect


def test_decode_noalloc_scratch_limit_is_the_header_constant(lib):
    text = open(HEADER).read()
    assert "#define ATTN_DECODE_NOALLOC_MAX_BYTES ((size_t)32 << 20)" in text
    assert attn.ATTN_DECODE_NOALLOC_MAX_BYTES == 32 << 20
    big = attn.attn_decode_workspace_size(8, 256, 8, 1, 128, 64, 131072)
    assert big > attn.ATTN_DECODE_NOALLOC_MAX_BYTES
    # the decode workloads all fit
    for args in ((8, 64, 8, 1, 128, 64, 131072, 0), (32, 32, 32, 1, 128, 16, 8192, 0),
                 (8, 64, 8, 4, 128, 256, 131072, 4096)):
        assert 0 < attn.attn_decode_workspace_size(*args) <= attn.ATTN_DECODE_NOALLOC_MAX_BYTES


@pytest.mark.parametrize("kw", [dict(B=0), dict(max_seq_len=0)])
def test_decode_noalloc_empty_problem_is_ok_and_launches_nothing(lib, kw):
    a = dict(NOALLOC_GOOD)
    a.update(kw)
    assert attn.attn_decode_paged_noalloc(**a) == attn.ATTN_OK


def test_decode_workspace_size(lib):
    n = attn.attn_decode_workspace_size(8, 64, 8, 1, 128, 64, 131072)
    assert attn.attn_decode_workspace_size(8, 64, 8, 1, 128, 64, 131072, 4096) < n
    assert n > 0 and n % 4 == 0
    # partial outputs (d floats) and lse (1 float) per (sequence, KV head, split, column)
    per = 8 * 8 * 8 * (128 + 1) * 4
    assert n % per == 0
    assert attn.attn_decode_workspace_size(0, 64, 8, 1, 128, 64, 1000) == 0
    assert attn.attn_decode_workspace_size(2, 64, 7, 1, 128, 64, 1000) == 0
    # the split never exceeds 64 page-table entries
    n16 = attn.attn_decode_workspace_size(1, 1, 1, 1, 64, 16, 1 << 20)
    assert n16 // ((64 + 1) * 4) >= (1 << 20) // (64 * 16)


@pytest.mark.parametrize("args,splits", [
    # 8 x 64/8 heads to 128k, pages of 64: 64 (sequence, KV head) groups, about
    # 4096 single-wave workgroups -> 64 splits of 2048 keys
    ((8, 64, 8, 1, 128, 64, 131072), 64),
    # 32 x 32 heads to 8k, pages of 16: the 64-entry page-table limit caps a
    # split at 1024 keys -> 8 splits
    ((32, 32, 32, 1, 128, 16, 8192), 8),
    # multi-query 8 x 64/1 heads to 128k: two 32-column blocks, splits of at
    # least 1024 keys (the measured best) -> 128 splits
    ((8, 64, 1, 1, 128, 64, 131072), 128),
    # 8 x 32/2 heads x 4 new tokens: 64 columns, 1024-key splits -> 128
    ((8, 32, 2, 4, 128, 64, 131072), 128),
])
def test_decode_split_plan_of_the_measured_workloads(lib, args, splits):
    """The split plan behind the decode workspace, worked out by hand: one
    partial O (d floats) and lse per (sequence, KV head, split, column)."""
    B, Hq, Hkv, T, d = args[:5]
    assert attn.attn_decode_workspace_size(*args) == B * Hkv * splits * (Hq // Hkv * T) * (d + 1) * 4


def test_decode_split_plan_with_a_window(lib):
    # window 4096, 4 new tokens, pages of 256: the span is the window plus the
    # new tokens plus one page of rounding (4355 keys); 64 groups want 64
    # splits, rounded up to whole pages: 18 splits of 256 keys
    assert attn.attn_decode_workspace_size(8, 64, 8, 4, 128, 256, 131072, 4096) == \
        8 * 8 * 18 * 32 * 129 * 4


VAR_GOOD = dict(q=P, k=P, v=P, o=P, lse=P, cu_seqlens=P, B=2, max_seqlen=64, total_rows=100, Hq=4,
                Hkv=2, d=128, scale=0.1, causal=0, window=0, radius=16, n_global=2)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(cu_seqlens=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(lse=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(B=-1), attn.ATTN_ERR_INVALID_ARG),
    (dict(total_rows=-1), attn.ATTN_ERR_INVALID_ARG),
    (dict(radius=-1), attn.ATTN_ERR_INVALID_ARG),
    (dict(n_global=-3), attn.ATTN_ERR_INVALID_ARG),
    (dict(Hq=3), attn.ATTN_ERR_INVALID_ARG),
    (dict(causal=5), attn.ATTN_ERR_INVALID_ARG),
    (dict(scale=float("inf")), attn.ATTN_ERR_INVALID_ARG),
    (dict(d=32), attn.ATTN_ERR_UNSUPPORTED),
    (dict(window=8), attn.ATTN_ERR_UNSUPPORTED),          # window needs causal
    (dict(cu_seqlens=P + 2), attn.ATTN_ERR_UNSUPPORTED),
    (dict(k=P + 8), attn.ATTN_ERR_UNSUPPORTED),
    (dict(max_seqlen=(1 << 22) + 1), attn.ATTN_ERR_UNSUPPORTED),
])
def test_varlen_rejects_bad_arguments_without_launching(lib, kw, expect):
    a = dict(VAR_GOOD)
    a.update(kw)
    assert attn.attn_fwd_varlen(**a) == expect


@pytest.mark.parametrize("kw", [dict(B=0), dict(max_seqlen=0), dict(total_rows=0),
                                dict(B=0, q=0, k=0, v=0, o=0, lse=0, cu_seqlens=0)])
def test_varlen_empty_problem_is_ok_and_launches_nothing(lib, kw):
    a = dict(VAR_GOOD)
    a.update(kw)
    assert attn.attn_fwd_varlen(**a) == attn.ATTN_OK


FP8Q_GOOD = dict(q=P, k=P, v=P, q8=P, k8=P, vt8=P, scales=P, B=1, Hq=4, Hkv=2, N=64, d=128)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(v=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(q8=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(k8=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(vt8=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(scales=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(B=-1), attn.ATTN_ERR_INVALID_ARG),
    (dict(Hq=6, Hkv=4), attn.ATTN_ERR_INVALID_ARG),
    (dict(d=32), attn.ATTN_ERR_UNSUPPORTED),
    (dict(k8=P + 2), attn.ATTN_ERR_UNSUPPORTED),
    (dict(vt8=P + 8), attn.ATTN_ERR_UNSUPPORTED),
    (dict(N=(1 << 22) + 1), attn.ATTN_ERR_UNSUPPORTED),
])
def test_fp8_quantize_rejects_bad_arguments_without_launching(lib, kw, expect):
    a = dict(FP8Q_GOOD)
    a.update(kw)
    assert attn.attn_fp8_quantize(**a) == expect


FP8F_GOOD = dict(q8=P, k8=P, vt8=P, scales=P, o=P, lse=P, B=1, Hq=4, Hkv=2, N=64, d=128,
                 scale=0.1, causal=1, window=0)


@pytest.mark.parametrize("kw,expect", [
    (dict(q8=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(vt8=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(scales=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(o=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(lse=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(Hq=6, Hkv=4), attn.ATTN_ERR_INVALID_ARG),
    (dict(causal=2), attn.ATTN_ERR_INVALID_ARG),
    (dict(scale=float("nan")), attn.ATTN_ERR_INVALID_ARG),
    (dict(d=96), attn.ATTN_ERR_UNSUPPORTED),
    (dict(causal=0, window=8), attn.ATTN_ERR_UNSUPPORTED),
    (dict(scales=P + 2), attn.ATTN_ERR_UNSUPPORTED),
    (dict(N=(1 << 22) + 1), attn.ATTN_ERR_UNSUPPORTED),
])
def test_fwd_fp8_rejects_bad_arguments_without_launching(lib, kw, expect):
    a = dict(FP8F_GOOD)
    a.update(kw)
    assert attn.attn_fwd_fp8(**a) == expect


@pytest.mark.parametrize("kw", [dict(B=0), dict(N=0),
                                dict(N=0, q8=0, k8=0, vt8=0, scales=0, o=0, lse=0)])
def test_fwd_fp8_empty_problem_is_ok_and_launches_nothing(lib, kw):
    a = dict(FP8F_GOOD)
    a.update(kw)
    assert attn.attn_fwd_fp8(**a) == attn.ATTN_OK


@pytest.mark.parametrize("kw", [dict(B=0), dict(N=0),
                                dict(B=0, q=0, k=0, v=0, q8=0, k8=0, vt8=0, scales=0)])
def test_fp8_quantize_empty_problem_is_ok_and_launches_nothing(lib, kw):
    a = dict(FP8Q_GOOD)
    a.update(kw)
    assert attn.attn_fp8_quantize(**a) == attn.ATTN_OK


def test_fp8_vt_bytes(lib):
    # V^T codes: d rows of the key count rounded up to 64, per (batch, KV head)
    assert attn.attn_fp8_vt_bytes(2, 8, 100, 128) == 2 * 8 * 128 * 128
    assert attn.attn_fp8_vt_bytes(1, 1, 64, 64) == 64 * 64
    assert attn.attn_fp8_vt_bytes(1, 1, 65, 64) == 64 * 128
    assert attn.attn_fp8_vt_bytes(0, 1, 64, 64) == 0
    assert attn.attn_fp8_vt_bytes(1, 1, 64, 96) == 0
