"""ctypes binding of libfa_mi355x.so (the C ABI in include/fa_mi355x.h).

Argument marshalling only: every step of the attention runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory and the current
stream.  The raw functions (``fa_fwd``, ``fa_fwd_f32``, ``fa_fwd_ex``,
``fa_fwd_splitkv``, ``fa_combine``) take the C arguments one to one; tensor
arguments may be torch tensors (their ``data_ptr()`` is passed) or integer
device addresses.  They raise :class:`FaError` on a non-zero status.

``attention`` and ``splitkv_attention`` allocate the outputs with torch and
call the raw functions with shapes taken from the tensors.

The library is loaded on first use.  If it is missing the call raises: there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libfa_mi355x.so"

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP = 0, -1, -2, -3
FA_DTYPE_BF16, FA_DTYPE_FP32 = 0, 1
FA_MAX_HEAD_WINDOWS = 256

EXPORTED = ("fa_fwd", "fa_fwd_f32", "fa_fwd_ex", "fa_fwd_fp8", "fa_fwd_splitkv", "fa_combine", "fa_kv_append",
            "fa_decode_rolling", "fa_softmax", "fa_softmax_topk", "fa_splitkv_attention_static", "fa_status_string")
FA_ERR_SCRATCH_LIMIT = -4
FA_STATIC_SCRATCH_BYTES = 8 << 20
FA_MAX_TOPK = 64


class FaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {fa_status_string(status)} ({status})")
        self.status = status


class FwdArgs(ctypes.Structure):
    """Mirror of struct fa_fwd_args."""
    _fields_ = [
        ("dtype", ctypes.c_int),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("B", ctypes.c_int64), ("H", ctypes.c_int64), ("Hkv", ctypes.c_int64),
        ("Nq", ctypes.c_int64), ("Nk", ctypes.c_int64), ("d", ctypes.c_int64),
        ("scale", ctypes.c_float),
        ("causal", ctypes.c_int),
        ("window", ctypes.c_int),
        ("softcap", ctypes.c_float),
        ("head_window", ctypes.POINTER(ctypes.c_int32)),
        ("stream", ctypes.c_void_p),
    ]


_lib = None


def library_path() -> str:
    return os.path.join(HERE, _LIB_NAME)


def load_library():
    """Load libfa_mi355x.so (once).  Raises FileNotFoundError if not built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is not built; run `python -m online_softmax_tiled_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i64, f32, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    fwd_args = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, f32, ci, ci, f32, vp]
    lib.fa_fwd.argtypes = fwd_args
    lib.fa_fwd_f32.argtypes = fwd_args
    lib.fa_fwd_ex.argtypes = [ctypes.POINTER(FwdArgs)]
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, f32, f32, f32, f32,
                               ci, ci, vp]
    lib.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                   f32, ci, ci, f32, ci, vp]
    lib.fa_combine.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ci, ci, vp]
    lib.fa_kv_append.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, vp]
    lib.fa_decode_rolling.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64,
                                      f32, f32, ci, vp]
    lib.fa_softmax.argtypes = [vp, vp, vp, i64, i64, ci, vp]
    lib.fa_softmax_topk.argtypes = [vp, vp, vp, vp, i64, i64, ci, ci, vp]
    lib.fa_splitkv_attention_static.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, f32, ci, ci,
                                                f32, ci, ci, vp]
    for name in ("fa_fwd", "fa_fwd_f32", "fa_fwd_ex", "fa_fwd_fp8", "fa_fwd_splitkv", "fa_combine", "fa_kv_append",
                 "fa_decode_rolling", "fa_softmax", "fa_softmax_topk", "fa_splitkv_attention_static"):
        getattr(lib, name).restype = ci
    lib.fa_status_string.argtypes = [ci]
    lib.fa_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x or None
    return x.data_ptr() or None


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream or None
    if isinstance(stream, int):
        return stream or None
    return stream.cuda_stream or None


def _check(status: int, what: str):
    if status != FA_OK:
        raise FaError(status, what)


# ------------------------------------------------------------------ raw ABI
def fa_fwd(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, window, softcap, stream=None):
    _check(load_library().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, Nq, Nk, d,
                                 float(scale), int(causal), int(window), float(softcap), _stream(stream)),
           "fa_fwd")


def fa_fwd_f32(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, window, softcap, stream=None):
    _check(load_library().fa_fwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, Nq, Nk, d,
                                     float(scale), int(causal), int(window), float(softcap), _stream(stream)),
           "fa_fwd_f32")


def fa_fwd_ex(dtype, q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, window, softcap,
              head_window=None, stream=None):
    hw = None
    if head_window is not None:
        # The library reads head_window[h] for every h < H.
        if len(head_window) != int(H):
            raise ValueError(f"head_window has {len(head_window)} entries; it needs one per query head (H={H})")
        hw = (ctypes.c_int32 * len(head_window))(*[int(x) for x in head_window])
    a = FwdArgs(int(dtype), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, Nq, Nk, d,
                float(scale), int(causal), int(window), float(softcap),
                ctypes.cast(hw, ctypes.POINTER(ctypes.c_int32)) if hw is not None else None,
                _stream(stream))
    _check(load_library().fa_fwd_ex(ctypes.byref(a)), "fa_fwd_ex")


def fa_fwd_splitkv(q, k, v, o_part, m_part, l_part, B, H, Hkv, Nq, Nk, d, scale, causal, window,
                   softcap, num_splits, stream=None):
    _check(load_library().fa_fwd_splitkv(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o_part), _ptr(m_part), _ptr(l_part), B, H, Hkv, Nq, Nk, d,
        float(scale), int(causal), int(window), float(softcap), int(num_splits), _stream(stream)),
        "fa_fwd_splitkv")


def fa_combine(o_part, m_part, l_part, o, lse, B, H, Nq, d, num_splits, out_dtype, stream=None):
    _check(load_library().fa_combine(_ptr(o_part), _ptr(m_part), _ptr(l_part), _ptr(o), _ptr(lse),
                                      B, H, Nq, d, int(num_splits), int(out_dtype), _stream(stream)),
           "fa_combine")


def fa_kv_append(k_new, v_new, k_cache, v_cache, B, Hkv, T, d, pos, window, sinks, stream=None):
    _check(load_library().fa_kv_append(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), B, Hkv, T, d,
                                        int(pos), int(window), int(sinks), _stream(stream)),
           "fa_kv_append")


def fa_decode_rolling(q, k_cache, v_cache, o_part, m_part, l_part, B, H, Hkv, d, pos, window, sinks, scale,
                      softcap, num_splits, stream=None):
    _check(load_library().fa_decode_rolling(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o_part), _ptr(m_part), _ptr(l_part), B, H, Hkv, d,
        int(pos), int(window), int(sinks), float(scale), float(softcap), int(num_splits), _stream(stream)),
        "fa_decode_rolling")


def fa_softmax(x, y, lse, rows, n, dtype, stream=None):
    _check(load_library().fa_softmax(_ptr(x), _ptr(y), _ptr(lse), rows, n, int(dtype), _stream(stream)),
           "fa_softmax")


def fa_softmax_topk(x, probs, indices, lse, rows, n, k, dtype, stream=None):
    _check(load_library().fa_softmax_topk(_ptr(x), _ptr(probs), _ptr(indices), _ptr(lse), rows, n, int(k),
                                           int(dtype), _stream(stream)),
           "fa_softmax_topk")

def fa_splitkv_attention_static(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, window, softcap, num_splits,
                                out_dtype, stream=None):
    _check(load_library().fa_splitkv_attention_static(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, Nq, Nk, d, float(scale), int(causal),
        int(window), float(softcap), int(num_splits), int(out_dtype), _stream(stream)),
        "fa_splitkv_attention_static")


def fa_fwd_fp8(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, q_descale, k_descale, v_descale, causal, window,
               stream=None):
    _check(load_library().fa_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, Nq, Nk, d,
                                     float(scale), float(q_descale), float(k_descale), float(v_descale),
                                     int(causal), int(window), _stream(stream)),
           "fa_fwd_fp8")


# ------------------------------------------------------------- conveniences
def _shapes(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D: [B, H, N, d]")
    B, H, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if Bk != B or dk != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError("q [B,H,Nq,d], k and v [B,Hkv,Nk,d] shapes disagree")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous device tensors")
        _check_aligned(t, 16, "q, k, v")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share one dtype")
    return B, H, Hkv, Nq, Nk, d


def _check_aligned(t, nbytes, name):
    """The kernels move 16 bytes per lane from and to the base of q, k, v, o
    and the partials (4 bytes for fp32 row arrays); a view that starts at an
    element offset may break that, and the library would refuse it."""
    if t.numel() and t.data_ptr() % nbytes:
        raise ValueError(f"{name} must start at a {nbytes}-byte aligned address (got a view at an offset)")


def _buffer(t, shape, dtype, device, name, align=16):
    """A caller-supplied output buffer: it must be a contiguous device tensor
    of exactly this shape and dtype (the kernels write every element of it
    and nothing past it)."""
    import torch
    shape = tuple(int(x) for x in shape)
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if tuple(t.shape) != shape or t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} device tensor of shape {list(shape)}, "
                         f"got {t.dtype} {list(t.shape)}")
    _check_aligned(t, align, name)
    return t


def attention(q, k, v, scale=None, causal=False, window=0, head_window=None, softcap=0.0,
              out=None, lse=None):
    """O = softmax(scale * q k^T) v per head (exact, tiled).  q: [B,H,Nq,d],
    k, v: [B,Hkv,Nk,d], bf16 or fp32 on the GPU.  Returns (o, lse)."""
    import torch
    B, H, Hkv, Nq, Nk, d = _shapes(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if q.dtype == torch.bfloat16:
        dtype = FA_DTYPE_BF16
    elif q.dtype == torch.float32:
        dtype = FA_DTYPE_FP32
    else:
        raise ValueError("q, k, v must be bfloat16 or float32")
    o = _buffer(out, q.shape, q.dtype, q.device, "out")
    lse = _buffer(lse, (B, H, Nq), torch.float32, q.device, "lse", align=4)
    if head_window is not None:
        fa_fwd_ex(dtype, q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, window, softcap,
                  head_window=head_window)
    elif dtype == FA_DTYPE_BF16:
        fa_fwd(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, window, softcap)
    else:
        fa_fwd_f32(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, window, softcap)
    return o, lse


def attention_fp8(q, k, v, q_descale=1.0, k_descale=1.0, v_descale=1.0, scale=None, causal=False, window=0,
                  out=None, lse=None):
    """fp8 attention: q [B,H,Nq,d], k, v [B,Hkv,Nk,d] hold OCP E4M3 bytes
    (torch.float8_e4m3fn or torch.uint8) whose values are multiplied by the
    descale factors.  Returns (o bf16 [B,H,Nq,d], lse fp32 [B,H,Nq])."""
    import torch
    if q.dtype not in (torch.float8_e4m3fn, torch.uint8):
        raise ValueError("q, k, v must be float8_e4m3fn or uint8 (E4M3 bytes)")
    B, H, Hkv, Nq, Nk, d = _shapes(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    o = _buffer(out, (B, H, Nq, d), torch.bfloat16, q.device, "out")
    lse = _buffer(lse, (B, H, Nq), torch.float32, q.device, "lse", align=4)
    fa_fwd_fp8(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, q_descale, k_descale, v_descale, causal, window)
    return o, lse


def splitkv_attention(q, k, v, num_splits, scale=None, causal=False, window=0, softcap=0.0,
                      out_dtype=None, partials=None, return_partials=False):
    """Split-KV attention: per-split partials (fa_fwd_splitkv) merged by
    fa_combine.  q, k, v bf16.  ``partials`` may pass preallocated
    (o_part [B,H,Nq,S,d], m_part, l_part [B,H,Nq,S]) fp32 buffers."""
    import torch
    B, H, Hkv, Nq, Nk, d = _shapes(q, k, v)
    if q.dtype != torch.bfloat16:
        raise ValueError("split-KV takes bfloat16 q, k, v")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    S = int(num_splits)
    o_part, m_part, l_part = (None, None, None) if partials is None else partials
    o_part = _buffer(o_part, (B, H, Nq, S, d), torch.float32, q.device, "o_part")
    m_part = _buffer(m_part, (B, H, Nq, S), torch.float32, q.device, "m_part", align=4)
    l_part = _buffer(l_part, (B, H, Nq, S), torch.float32, q.device, "l_part", align=4)
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    o = torch.empty((B, H, Nq, d), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    fa_fwd_splitkv(q, k, v, o_part, m_part, l_part, B, H, Hkv, Nq, Nk, d, scale, causal, window,
                   softcap, S)
    fa_combine(o_part, m_part, l_part, o, lse, B, H, Nq, d, S,
               FA_DTYPE_BF16 if out_dtype == torch.bfloat16 else FA_DTYPE_FP32)
    if return_partials:
        return o, lse, (o_part, m_part, l_part)
    return o, lse


class RollingKVCache:
    """One layer's rolling KV cache for streaming decode: ``sinks`` rows that
    keep the first tokens, then a ring of ``window`` rows for the most recent
    ones (bf16 [B, Hkv, sinks + window, d] each, allocated with torch).
    ``append`` writes the next tokens' K/V (fa_kv_append); ``attend`` runs
    fa_decode_rolling + fa_combine for the query of the last written token."""

    def __init__(self, B, Hkv, d, window, sinks=4, device="cuda"):
        import torch
        self.B, self.Hkv, self.d, self.window, self.sinks = int(B), int(Hkv), int(d), int(window), int(sinks)
        shape = (self.B, self.Hkv, self.sinks + self.window, self.d)
        self.k = torch.zeros(shape, dtype=torch.bfloat16, device=device)
        self.v = torch.zeros(shape, dtype=torch.bfloat16, device=device)
        self.length = 0  # tokens written so far (positions 0 .. length-1)

    def append(self, k_new, v_new, stream=None):
        """k_new, v_new: bf16 [B, Hkv, T, d], the tokens at positions
        length .. length+T-1."""
        B, Hkv, T, d = k_new.shape
        if (B, Hkv, d) != (self.B, self.Hkv, self.d) or v_new.shape != k_new.shape:
            raise ValueError("k_new / v_new shape does not match the cache")
        fa_kv_append(k_new, v_new, self.k, self.v, B, Hkv, T, d, self.length, self.window, self.sinks, stream)
        self.length += T

    def attend(self, q, num_splits=4, scale=None, softcap=0.0, out_dtype=None, stream=None):
        """Attention of q (bf16 [B, H, 1, d]), the query of the token at
        position length-1, over the sink tokens and the window."""
        import torch
        if self.length < 1:
            raise ValueError("the cache is empty")
        B, H, Nq, d = q.shape
        if Nq != 1 or B != self.B or d != self.d:
            raise ValueError("q must be [B, H, 1, d] for this cache")
        scale = 1.0 / math.sqrt(d) if scale is None else scale
        S = int(num_splits)
        o_part = torch.empty((B, H, 1, S, d), dtype=torch.float32, device=q.device)
        m_part = torch.empty((B, H, 1, S), dtype=torch.float32, device=q.device)
        l_part = torch.empty((B, H, 1, S), dtype=torch.float32, device=q.device)
        out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
        o = torch.empty((B, H, 1, d), dtype=out_dtype, device=q.device)
        lse = torch.empty((B, H, 1), dtype=torch.float32, device=q.device)
        fa_decode_rolling(q, self.k, self.v, o_part, m_part, l_part, B, H, self.Hkv, d, self.length - 1,
                          self.window, self.sinks, scale, softcap, S, stream)
        fa_combine(o_part, m_part, l_part, o, lse, B, H, 1, d, S,
                   FA_DTYPE_BF16 if out_dtype == torch.bfloat16 else FA_DTYPE_FP32, stream)
        return o, lse


def _rows_dtype(x):
    import torch
    if x.dtype not in (torch.float32, torch.bfloat16) or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous fp32 or bf16 CUDA tensor")
    n = x.shape[-1] if x.dim() else 1
    rows = x.numel() // n if n else 0
    return rows, n, FA_DTYPE_BF16 if x.dtype == torch.bfloat16 else FA_DTYPE_FP32


def softmax(x, return_lse=False, stream=None):
    """Softmax over the last axis of x (fp32 or bf16, same dtype out) with the
    online normaliser (fa_softmax)."""
    import torch
    rows, n, dt = _rows_dtype(x)
    y = torch.empty_like(x)
    lse = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device) if return_lse else None
    fa_softmax(x, y, lse, rows, n, dt, stream)
    return (y, lse) if return_lse else y


def softmax_topk(x, k, return_lse=False, stream=None):
    """The k largest softmax probabilities over the last axis of x and their
    indices (descending; equal values lower index first), from one read of x
    (fa_softmax_topk).  Returns (probs fp32 [..., k], indices int32 [..., k])."""
    import torch
    rows, n, dt = _rows_dtype(x)
    probs = torch.empty(x.shape[:-1] + (k,), dtype=torch.float32, device=x.device)
    idx = torch.empty(x.shape[:-1] + (k,), dtype=torch.int32, device=x.device)
    lse = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device) if return_lse else None
    fa_softmax_topk(x, probs, idx, lse, rows, n, k, dt, stream)
    return (probs, idx, lse) if return_lse else (probs, idx)
