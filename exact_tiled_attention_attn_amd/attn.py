"""Python binding of libattn.so (ctypes).  Argument marshalling only.

The names mirror include/attn.h.  Every step of the attention forward and
backward runs in the HIP library; PyTorch is used here for device memory and the current
stream.  There is no fallback: if the library is missing or a call fails, an
``AttnError`` is raised.
"""

from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn.so")

ATTN_OK = 0
ATTN_ERR_INVALID_ARG = 1
ATTN_ERR_UNSUPPORTED = 2
ATTN_ERR_LAUNCH = 3
ATTN_ERR_NO_SCRATCH = 4
ATTN_MAX_N = 1 << 22
ATTN_DECODE_NOALLOC_MAX_BYTES = 32 << 20

EXPORTED = ("attn_fwd", "attn_fwd_ex", "attn_fwd_varlen", "attn_fwd_fp8", "attn_fp8_quantize",
            "attn_fp8_vt_bytes", "attn_bwd", "attn_bwd_workspace_size",
            "attn_decode_paged", "attn_decode_workspace_size", "attn_decode_paged_noalloc",
            "attn_num_variants",
            "attn_variant_name", "attn_status_string", "attn_device_info", "attn_abi_version")


class AttnError(RuntimeError):
    """The library is missing or returned a non-OK status."""

    def __init__(self, msg, status=None):
        super().__init__(msg)
        self.status = status


_lib = None


def load_library():
    """Load libattn.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise AttnError(f"{LIB_PATH} is not built; run "
                        "`python -m exact_tiled_attention_attn_amd.build` first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
    lib.attn_fwd.restype = i
    lib.attn_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp]
    lib.attn_fwd_ex.restype = i
    lib.attn_fwd_varlen.argtypes = [vp] * 6 + [i] * 6 + [f, i, i, i, i, vp]
    lib.attn_fwd_varlen.restype = i
    lib.attn_fp8_vt_bytes.argtypes = [i] * 4
    lib.attn_fp8_vt_bytes.restype = ctypes.c_size_t
    lib.attn_fp8_quantize.argtypes = [vp] * 7 + [i] * 5 + [vp]
    lib.attn_fp8_quantize.restype = i
    lib.attn_fwd_fp8.argtypes = [vp] * 6 + [i] * 5 + [f, i, i, vp]
    lib.attn_fwd_fp8.restype = i
    lib.attn_bwd.argtypes = [vp] * 10 + [i, i, i, i, i, f, i, i, vp]
    lib.attn_bwd.restype = i
    lib.attn_bwd_workspace_size.argtypes = [i, i, i]
    lib.attn_bwd_workspace_size.restype = ctypes.c_size_t
    lib.attn_decode_paged.argtypes = [vp] * 8 + [i] * 9 + [f, i, vp]
    lib.attn_decode_paged.restype = i
    lib.attn_decode_workspace_size.argtypes = [i] * 8
    lib.attn_decode_workspace_size.restype = ctypes.c_size_t
    lib.attn_decode_paged_noalloc.argtypes = [vp] * 7 + [i] * 9 + [f, i, vp]
    lib.attn_decode_paged_noalloc.restype = i
    lib.attn_num_variants.argtypes = []
    lib.attn_num_variants.restype = i
    lib.attn_variant_name.argtypes = [i]
    lib.attn_variant_name.restype = ctypes.c_char_p
    lib.attn_status_string.argtypes = [i]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_device_info.argtypes = [i] + [ctypes.POINTER(i)] * 4
    lib.attn_device_info.restype = i
    lib.attn_abi_version.argtypes = []
    lib.attn_abi_version.restype = i
    _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x or None
    return x.data_ptr() or None


def _stream(stream, *tensors):
    if stream is None:
        if any(getattr(t, "is_cuda", False) for t in tensors):
            import torch
            return torch.cuda.current_stream().cuda_stream or None
        return None
    if isinstance(stream, int):
        return stream or None
    return stream.cuda_stream or None


def _check_out(t, shape, dtype, device, name):
    """A caller-supplied output buffer must have exactly the shape, dtype and
    device the call writes, and be contiguous (the kernels write it densely)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise AttnError(f"{name} must be a tensor")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device:
        raise AttnError(f"{name} must be {tuple(shape)} {dtype} on {device}, "
                        f"got {tuple(t.shape)} {t.dtype} on {t.device}")
    if not t.is_contiguous():
        raise AttnError(f"{name} must be contiguous")


def _check_workspace(ws, nbytes, device, name="workspace"):
    """A caller-supplied workspace must hold at least the bytes the C side
    asks for (the C entry point cannot check the size it is given)."""
    import torch
    if not isinstance(ws, torch.Tensor) or ws.device != device or not ws.is_contiguous():
        raise AttnError(f"{name} must be a contiguous tensor on {device}")
    have = ws.numel() * ws.element_size()
    if have < nbytes:
        raise AttnError(f"{name} holds {have} bytes, the call needs {nbytes}")


def attn_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, window, stream=None):
    """Call the C entry point; returns its status code (0 = ATTN_OK).

    q, k, v, o, lse: torch tensors or raw device addresses (int).
    stream: torch stream, raw hipStream_t (int) or None for the current
    torch stream.
    """
    lib = load_library()
    return lib.attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(Hq),
                        int(Hkv), int(N), int(d), float(scale), int(causal), int(window),
                        _stream(stream, q, k, v, o, lse))


def attn_fwd_ex(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, window, variant,
                stream=None):
    """attn_fwd with an explicit kernel variant id; returns the status code."""
    lib = load_library()
    return lib.attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(Hq),
                           int(Hkv), int(N), int(d), float(scale), int(causal), int(window),
                           int(variant), _stream(stream, q, k, v, o, lse))


def attn_fwd_varlen(q, k, v, o, lse, cu_seqlens, B, max_seqlen, total_rows, Hq, Hkv, d, scale,
                    causal, window, radius, n_global, stream=None):
    """Call the C packed-sequence forward; returns its status code."""
    lib = load_library()
    return lib.attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens),
                               int(B), int(max_seqlen), int(total_rows), int(Hq), int(Hkv),
                               int(d), float(scale), int(causal), int(window), int(radius),
                               int(n_global), _stream(stream, q, k, v, o, lse))


def attn_fp8_vt_bytes(B, Hkv, N, d):
    return int(load_library().attn_fp8_vt_bytes(int(B), int(Hkv), int(N), int(d)))


def attn_fp8_quantize(q, k, v, q8, k8, vt8, scales, B, Hq, Hkv, N, d, stream=None):
    lib = load_library()
    return lib.attn_fp8_quantize(_ptr(q), _ptr(k), _ptr(v), _ptr(q8), _ptr(k8), _ptr(vt8),
                                 _ptr(scales), int(B), int(Hq), int(Hkv), int(N), int(d),
                                 _stream(stream, q, k, v, q8, k8, vt8, scales))


def attn_fwd_fp8(q8, k8, vt8, scales, o, lse, B, Hq, Hkv, N, d, scale, causal, window,
                 stream=None):
    lib = load_library()
    return lib.attn_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(vt8), _ptr(scales), _ptr(o), _ptr(lse),
                            int(B), int(Hq), int(Hkv), int(N), int(d), float(scale), int(causal),
                            int(window), _stream(stream, q8, k8, vt8, scales, o, lse))


def attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, Hq, Hkv, N, d, scale, causal,
             window, stream=None):
    """Call the C backward entry point; returns its status code (0 = ATTN_OK).

    Tensors or raw device addresses (int), as for attn_fwd.
    """
    lib = load_library()
    return lib.attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                        _ptr(dk), _ptr(dv), _ptr(workspace), int(B), int(Hq), int(Hkv), int(N),
                        int(d), float(scale), int(causal), int(window),
                        _stream(stream, q, k, v, o, lse, dout, dq, dk, dv))


def attn_bwd_workspace_size(B, Hq, N):
    return int(load_library().attn_bwd_workspace_size(int(B), int(Hq), int(N)))


def attn_decode_paged(q, k_cache, v_cache, block_table, seq_lens, o, lse, workspace, B, Hq, Hkv,
                      T, d, page_size, num_pages, max_pages_per_seq, max_seq_len, scale, window,
                      stream=None):
    """Call the C paged-decode entry point; returns its status code."""
    lib = load_library()
    return lib.attn_decode_paged(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens), _ptr(o),
        _ptr(lse), _ptr(workspace), int(B), int(Hq), int(Hkv), int(T), int(d), int(page_size),
        int(num_pages), int(max_pages_per_seq), int(max_seq_len), float(scale), int(window),
        _stream(stream, q, k_cache, v_cache, o, lse))


def attn_decode_paged_noalloc(q, k_cache, v_cache, block_table, seq_lens, o, lse, B, Hq, Hkv,
                              T, d, page_size, num_pages, max_pages_per_seq, max_seq_len, scale,
                              window, stream=None):
    """Call the C allocation-free paged-decode entry point; returns its status."""
    lib = load_library()
    return lib.attn_decode_paged_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens), _ptr(o),
        _ptr(lse), int(B), int(Hq), int(Hkv), int(T), int(d), int(page_size), int(num_pages),
        int(max_pages_per_seq), int(max_seq_len), float(scale), int(window),
        _stream(stream, q, k_cache, v_cache, o, lse))


def attn_decode_workspace_size(B, Hq, Hkv, T, d, page_size, max_seq_len, window=0):
    return int(load_library().attn_decode_workspace_size(int(B), int(Hq), int(Hkv), int(T),
                                                         int(d), int(page_size),
                                                         int(max_seq_len), int(window)))


def attn_num_variants():
    return load_library().attn_num_variants()


def attn_variant_name(variant):
    return load_library().attn_variant_name(int(variant)).decode()


def attn_status_string(status):
    return load_library().attn_status_string(int(status)).decode()


def attn_device_info(device=0):
    """(compute units, peak engine clock kHz, memory clock kHz, bus bits)."""
    vals = [ctypes.c_int(0) for _ in range(4)]
    st = load_library().attn_device_info(int(device), *[ctypes.byref(x) for x in vals])
    if st != ATTN_OK:
        raise AttnError(f"attn_device_info: {attn_status_string(st)}", st)
    return tuple(x.value for x in vals)


def attn_abi_version():
    return load_library().attn_abi_version()


def fwd(q, k, v, causal=False, window=0, scale=None, variant=0, out=None, stream=None):
    """Allocate (o, lse) with torch and run the forward; raises on any error.

    q: (B, Hq, N, d) bf16 CUDA tensor, contiguous; k, v: (B, Hkv, N, d).
    Returns o (B, Hq, N, d) bf16 and lse (B, Hq, N) fp32.
    """
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise AttnError(f"{name} must be a CUDA (HIP) tensor")
        if t.dtype != torch.bfloat16:
            raise AttnError(f"{name} must be bfloat16")
        if not t.is_contiguous():
            raise AttnError(f"{name} must be contiguous")
        if t.dim() != 4:
            raise AttnError(f"{name} must be (B, H, N, d)")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, N, d) or tuple(v.shape) != tuple(k.shape):
        raise AttnError("k and v must be (B, Hkv, N, d) matching q")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        _check_out(o, q.shape, torch.bfloat16, q.device, "o")
        _check_out(lse, (B, Hq, N), torch.float32, q.device, "lse")
    st = attn_fwd_ex(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, int(bool(causal)), int(window),
                     variant, stream)
    if st != ATTN_OK:
        raise AttnError(f"attn_fwd failed: {attn_status_string(st)} (status {st})", st)
    return o, lse


def bwd(q, k, v, o, lse, dout, causal=False, window=0, scale=None, out=None, workspace=None,
        stream=None):
    """Allocate (dq, dk, dv) and the workspace with torch and run the backward.

    q, k, v, o, lse: as passed to / returned by ``fwd`` for the same
    arguments; dout: (B, Hq, N, d) bf16.  Returns (dq, dk, dv) in bf16 with
    the shapes of q, k and v.  Raises on any error.
    """
    import torch
    for name, t, dt in (("q", q, torch.bfloat16), ("k", k, torch.bfloat16),
                        ("v", v, torch.bfloat16), ("o", o, torch.bfloat16),
                        ("dout", dout, torch.bfloat16), ("lse", lse, torch.float32)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise AttnError(f"{name} must be a CUDA (HIP) tensor")
        if t.dtype != dt:
            raise AttnError(f"{name} must be {dt}")
        if not t.is_contiguous():
            raise AttnError(f"{name} must be contiguous")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if (tuple(k.shape) != (B, Hkv, N, d) or tuple(v.shape) != tuple(k.shape)
            or tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape)
            or tuple(lse.shape) != (B, Hq, N)):
        raise AttnError("shapes must be q, o, dout (B, Hq, N, d), k, v (B, Hkv, N, d), "
                        "lse (B, Hq, N)")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = out
        _check_out(dq, q.shape, torch.bfloat16, q.device, "dq")
        _check_out(dk, k.shape, torch.bfloat16, q.device, "dk")
        _check_out(dv, v.shape, torch.bfloat16, q.device, "dv")
    nbytes = attn_bwd_workspace_size(B, Hq, N)
    if workspace is None:
        workspace = torch.empty((max(nbytes, 4) // 4,), dtype=torch.float32, device=q.device)
    else:
        _check_workspace(workspace, nbytes, q.device)
    st = attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, Hq, Hkv, N, d, scale,
                  int(bool(causal)), int(window), stream)
    if st != ATTN_OK:
        raise AttnError(f"attn_bwd failed: {attn_status_string(st)} (status {st})", st)
    return dq, dk, dv


def decode(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, window=0, scale=None,
           out=None, workspace=None, stream=None):
    """Paged decode: allocate (o, lse) and the workspace with torch; raises on
    any error.

    q: (B, Hq, T, d) bf16; k_cache, v_cache: (num_pages, page_size, Hkv, d)
    bf16; block_table: (B, max_pages) int32; seq_lens: (B,) int32 (device).
    Returns o (B, Hq, T, d) bf16 and lse (B, Hq, T) fp32.
    """
    import torch
    for name, t, dt in (("q", q, torch.bfloat16), ("k_cache", k_cache, torch.bfloat16),
                        ("v_cache", v_cache, torch.bfloat16),
                        ("block_table", block_table, torch.int32),
                        ("seq_lens", seq_lens, torch.int32)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise AttnError(f"{name} must be a CUDA (HIP) tensor")
        if t.dtype != dt:
            raise AttnError(f"{name} must be {dt}")
        if not t.is_contiguous():
            raise AttnError(f"{name} must be contiguous")
    if q.dim() != 4 or k_cache.dim() != 4 or block_table.dim() != 2 or seq_lens.dim() != 1:
        raise AttnError("q (B, Hq, T, d), caches (pages, page_size, Hkv, d), "
                        "block_table (B, max_pages), seq_lens (B,)")
    B, Hq, T, d = q.shape
    num_pages, page_size, Hkv, dk = k_cache.shape
    if (tuple(v_cache.shape) != tuple(k_cache.shape) or dk != d or block_table.shape[0] != B
            or seq_lens.shape[0] != B):
        raise AttnError("shapes do not match")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        _check_out(o, q.shape, torch.bfloat16, q.device, "o")
        _check_out(lse, (B, Hq, T), torch.float32, q.device, "lse")
    nbytes = attn_decode_workspace_size(B, Hq, Hkv, T, d, page_size, max_seq_len,
                                        max(int(window), 0))
    if workspace is None:
        workspace = torch.empty((max(nbytes, 16) // 4,), dtype=torch.float32, device=q.device)
    else:
        _check_workspace(workspace, nbytes, q.device)
    st = attn_decode_paged(q, k_cache, v_cache, block_table, seq_lens, o, lse, workspace, B, Hq,
                           Hkv, T, d, page_size, num_pages, block_table.shape[1], max_seq_len,
                           scale, int(window), stream)
    if st != ATTN_OK:
        raise AttnError(f"attn_decode_paged failed: {attn_status_string(st)} (status {st})", st)
    return o, lse


def fwd_varlen(q, k, v, cu_seqlens, max_seqlen, causal=False, window=0, radius=0, n_global=0,
               scale=None, out=None, stream=None):
    """Packed-sequence forward with structured masks; raises on any error.

    q: (Hq, total, d) bf16; k, v: (Hkv, total, d) bf16; cu_seqlens: (B + 1,)
    int32 on the device.  Returns o (Hq, total, d) bf16 and lse (Hq, total)
    fp32.
    """
    import torch
    for name, t, dt in (("q", q, torch.bfloat16), ("k", k, torch.bfloat16),
                        ("v", v, torch.bfloat16), ("cu_seqlens", cu_seqlens, torch.int32)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise AttnError(f"{name} must be a CUDA (HIP) tensor")
        if t.dtype != dt:
            raise AttnError(f"{name} must be {dt}")
        if not t.is_contiguous():
            raise AttnError(f"{name} must be contiguous")
    if q.dim() != 3 or k.dim() != 3 or cu_seqlens.dim() != 1:
        raise AttnError("q (Hq, total, d), k, v (Hkv, total, d), cu_seqlens (B + 1,)")
    Hq, total, d = q.shape
    Hkv = k.shape[0]
    if tuple(k.shape) != (Hkv, total, d) or tuple(v.shape) != tuple(k.shape):
        raise AttnError("k and v must be (Hkv, total, d) matching q")
    B = cu_seqlens.shape[0] - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((Hq, total), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        _check_out(o, q.shape, torch.bfloat16, q.device, "o")
        _check_out(lse, (Hq, total), torch.float32, q.device, "lse")
    st = attn_fwd_varlen(q, k, v, o, lse, cu_seqlens, B, max_seqlen, total, Hq, Hkv, d, scale,
                         int(bool(causal)), int(window), int(radius), int(n_global), stream)
    if st != ATTN_OK:
        raise AttnError(f"attn_fwd_varlen failed: {attn_status_string(st)} (status {st})", st)
    return o, lse


def fp8_quantize(q, k, v, stream=None):
    """Pack bf16 (B, H, N, d) q, k, v for attn_fwd_fp8.  Returns
    (q8, k8, vt8, scales) as uint8 / float32 CUDA tensors; raises on error."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.bfloat16 \
                or not t.is_contiguous() or t.dim() != 4:
            raise AttnError(f"{name} must be a contiguous (B, H, N, d) bf16 CUDA tensor")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    q8 = torch.empty(q.shape, dtype=torch.uint8, device=q.device)
    k8 = torch.empty(k.shape, dtype=torch.uint8, device=q.device)
    vt8 = torch.empty((max(attn_fp8_vt_bytes(B, Hkv, N, d), 16),), dtype=torch.uint8,
                      device=q.device)
    scales = torch.empty((8,), dtype=torch.float32, device=q.device)
    st = attn_fp8_quantize(q, k, v, q8, k8, vt8, scales, B, Hq, Hkv, N, d, stream)
    if st != ATTN_OK:
        raise AttnError(f"attn_fp8_quantize failed: {attn_status_string(st)} (status {st})", st)
    return q8, k8, vt8, scales


def fwd_fp8(q8, k8, vt8, scales, causal=False, window=0, scale=None, out=None, stream=None):
    """FP8 forward over fp8_quantize's outputs; returns (o bf16, lse fp32)."""
    import torch
    B, Hq, N, d = q8.shape
    Hkv = k8.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        o = torch.empty((B, Hq, N, d), dtype=torch.bfloat16, device=q8.device)
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q8.device)
    else:
        o, lse = out
        _check_out(o, (B, Hq, N, d), torch.bfloat16, q8.device, "o")
        _check_out(lse, (B, Hq, N), torch.float32, q8.device, "lse")
    st = attn_fwd_fp8(q8, k8, vt8, scales, o, lse, B, Hq, Hkv, N, d, scale, int(bool(causal)),
                      int(window), stream)
    if st != ATTN_OK:
        raise AttnError(f"attn_fwd_fp8 failed: {attn_status_string(st)} (status {st})", st)
    return o, lse
