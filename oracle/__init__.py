"""Plain fp64 CPU oracle for exact softmax attention and the split merge.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers.  Nothing in the GPU
library imports, links or runs anything here, and this package imports
nothing from it.

The arithmetic lives in ``oracle.c`` (compiled with gcc, no fast-math);
this module only builds it and marshals numpy arrays.  Every function
takes numpy arrays in the layouts

    q [B, H, Nq, d],  k, v [B, Hkv, Nk, d],  o [B, H, Nq, d],  lse [B, H, Nq]

and returns float64 results.  Citations of the pages are in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(out: str = _LIB, src: str = _SRC, extra: tuple = ()) -> str:
    """Compile the oracle with gcc (-O2, strict IEEE: no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
           "-fno-fast-math", "-ffp-contract=off", *extra, "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.oracle_attention.restype = ctypes.c_int
    lib.oracle_attention.argtypes = [
        dp, dp, dp, dp, dp, dp, dp,
        i64, i64, i64, i64, i64, i64,
        ctypes.c_double, ctypes.c_int, ctypes.POINTER(ctypes.c_int32), ctypes.c_double,
        i64, i64, i64, ctypes.POINTER(i64), i64, i64, ctypes.c_int]
    lib.oracle_combine.restype = ctypes.c_int
    lib.oracle_combine.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64]
    return lib


def load_variant(path: str):
    """Load another build of oracle.c (used by the planted-mistake tests)."""
    return _bind(ctypes.CDLL(path))


def _ptr(a, ctype=ctypes.c_double):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def attention(q, k, v, scale: float, causal: bool = False, window: int = 0,
              head_window=None, softcap: float = 0.0, rows=None,
              key_range=None, tile: int = 0, nthreads: int | None = None,
              lib=None, sinks: int = 0):
    """Exact attention of every row (or of the listed ``rows``).

    ``head_window`` (int sequence of length H) overrides ``window`` per query
    head.  ``rows`` are flat indices r = (b*H + h)*Nq + i.  ``key_range``
    (lo, hi) restricts the keys, as one split of the key axis does.
    ``tile`` > 0 runs the streaming recurrence with that many keys per tile
    instead of the direct definition.  ``sinks`` > 0 keeps keys j < sinks
    visible to windowed rows (attention sinks, Transformers & Math 16.6).

    Returns dict(o, lse, m, l): o is [B,H,Nq,d] (or [len(rows), d]); lse, m
    and l are [B,H,Nq] (or [len(rows)]); m and l are the row maximum and the
    sum of exp(s - m), the per-block state of the merge equations.
    """
    lib = lib or _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if Bk != B or dk != d or v.shape != k.shape:
        raise ValueError("shape mismatch between q, k and v")
    hw = np.full(H, int(window), dtype=np.int32) if head_window is None else \
        np.ascontiguousarray(np.asarray(head_window, dtype=np.int32))
    if hw.shape != (H,):
        raise ValueError("head_window must have one entry per query head")
    lo, hi = (0, Nk) if key_range is None else key_range
    if rows is None:
        rows_arr, n = None, B * H * Nq
        oshape, rshape = (B, H, Nq, d), (B, H, Nq)
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = rows_arr.size
        oshape, rshape = (n, d), (n,)
    o = np.empty(oshape, dtype=np.float64)
    lse = np.empty(rshape, dtype=np.float64)
    m = np.empty(rshape, dtype=np.float64)
    ell = np.empty(rshape, dtype=np.float64)
    rc = lib.oracle_attention(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(m), _ptr(ell),
        B, H, Hkv, Nq, Nk, d, float(scale), int(bool(causal)), _ptr(hw, ctypes.c_int32),
        float(softcap), int(sinks), int(lo), int(hi),
        _ptr(rows_arr, ctypes.c_int64), n, int(tile),
        int(nthreads if nthreads is not None else default_threads()))
    if rc != 0:
        raise ValueError(f"oracle_attention rejected its arguments (rc={rc})")
    return {"o": o, "lse": lse, "m": m, "l": ell}


def split_partials(q, k, v, scale: float, num_splits: int, causal: bool = False,
                   window: int = 0, head_window=None, softcap: float = 0.0,
                   nthreads: int | None = None, lib=None):
    """Per-split results for keys cut into ``num_splits`` chunks of
    ceil(Nk / num_splits) keys: o_part [B,H,Nq,S,d] (each split's own
    normalised output), m_part and l_part [B,H,Nq,S]."""
    B, H, Nq, d = np.shape(q)
    Nk = np.shape(k)[2]
    chunk = -(-Nk // num_splits) if Nk > 0 else 0
    o_part = np.zeros((B, H, Nq, num_splits, d))
    m_part = np.full((B, H, Nq, num_splits), -np.inf)
    l_part = np.zeros((B, H, Nq, num_splits))
    for s in range(num_splits):
        lo, hi = min(Nk, s * chunk), min(Nk, (s + 1) * chunk)
        r = attention(q, k, v, scale, causal, window, head_window, softcap,
                      key_range=(lo, hi), nthreads=nthreads, lib=lib)
        o_part[:, :, :, s, :] = r["o"]
        m_part[:, :, :, s] = r["m"]
        l_part[:, :, :, s] = r["l"]
    return o_part, m_part, l_part


def combine(o_part, m_part, l_part, lib=None):
    """Merge per-split (O_s, m_s, l_s) of shape [..., S, d] / [..., S] into
    (o [..., d], lse [...])."""
    lib = lib or _load()
    o_part, m_part, l_part = _f64(o_part), _f64(m_part), _f64(l_part)
    *lead, S, d = o_part.shape
    R = int(np.prod(lead)) if lead else 1
    if tuple(m_part.shape) != (*lead, S) or l_part.shape != m_part.shape:
        raise ValueError("partial shapes disagree")
    o = np.empty((*lead, d), dtype=np.float64)
    lse = np.empty(tuple(lead), dtype=np.float64)
    rc = lib.oracle_combine(_ptr(o_part), _ptr(m_part), _ptr(l_part), _ptr(o), _ptr(lse), R, S, d)
    if rc != 0:
        raise ValueError(f"oracle_combine rejected its arguments (rc={rc})")
    return o, lse
