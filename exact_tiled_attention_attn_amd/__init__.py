"""MI355X-native exact tiled attention: forward, backward and paged decode
(bf16, causal / window / GQA).

The compute path is the HIP library ``libattn.so`` built from ``csrc/`` and
loaded by :mod:`exact_tiled_attention_attn_amd.attn`.  Importing this package
does not load it; the first use of ``attn_fwd`` (or ``fwd``) does, and fails
loudly if the library has not been built.
"""

__all__ = ["attn_fwd", "attn_fwd_ex", "attn_fwd_varlen", "fwd_varlen", "attn_fwd_fp8",
           "attn_fp8_quantize", "fp8_quantize", "fwd_fp8", "attn_bwd", "attn_bwd_workspace_size",
           "attn_decode_paged", "attn_decode_workspace_size", "attn_status_string", "fwd",
           "bwd", "decode", "AttnError"]


def __getattr__(name):
    if name in __all__:
        from . import attn as _attn
        return getattr(_attn, name)
    raise AttributeError(name)
