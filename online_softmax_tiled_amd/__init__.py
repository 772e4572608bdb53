"""Exact tiled softmax attention (FlashAttention-style forward) for MI355X.

The compute path is the HIP library ``libfa_mi355x.so`` built from
``csrc/``; :mod:`online_softmax_tiled_amd.fa` binds its C ABI.  The library
is loaded on first use and every entry point raises if it is missing.
"""
from .fa import (  # noqa: F401
    FaError,
    RollingKVCache,
    attention,
    attention_fp8,
    fa_combine,
    fa_decode_rolling,
    fa_fwd,
    fa_fwd_ex,
    fa_fwd_f32,
    fa_fwd_fp8,
    fa_fwd_splitkv,
    fa_kv_append,
    fa_softmax,
    fa_softmax_topk,
    fa_status_string,
    library_path,
    load_library,
    softmax,
    softmax_topk,
    splitkv_attention,
)
