"""fp8 (OCP E4M3) inputs for the attention oracle, in plain fp64 numpy.

TEST INFRASTRUCTURE ONLY (like the rest of this package): the test suite,
the smoke check and the benchmark's CPU-baseline leg are the only callers;
the GPU library shares nothing with it.

The fp8 variant of tiled attention runs both products of the loop on
narrow operands while the online-softmax state stays wide (HiFA4, abstract,
with 4-bit operands on Ascend NPUs; the GPU library uses 8-bit E4M3).  What
it computes, up to the rounding of the weights, is exact attention of the
dequantised inputs

    q = q_descale * E4M3(q bytes),  k = k_descale * E4M3(k bytes),
    v = v_descale * E4M3(v bytes),

so the oracle decodes the bytes and hands the values to the fp64 attention
oracle (``oracle.attention``).  Every decoded value times an fp32 descale is
exact in fp64 (4 + 24 significant bits).

E4M3 as defined by the OCP 8-bit floating point specification: bit 7 sign,
bits 6..3 exponent field E (bias 7), bits 2..0 mantissa M.  E > 0:
(-1)^s * 2^(E-7) * (1 + M/8); E = 0: (-1)^s * 2^-6 * M/8 (subnormals); the
codes with E = 15 and M = 7 (0x7f, 0xff) are NaN; there are no infinities,
so the largest finite value is 2^8 * 1.75 = 448.
"""
from __future__ import annotations

import numpy as np

from . import attention as _attention


def e4m3_value(codes):
    """float64 values of E4M3 bytes (any integer array of codes 0..255)."""
    c = np.asarray(codes).astype(np.int64)
    if np.any((c < 0) | (c > 255)):
        raise ValueError("E4M3 codes are bytes")
    sign = np.where(c >= 128, -1.0, 1.0)
    e = (c >> 3) & 15
    mant = (c & 7).astype(np.float64)
    normal = np.ldexp(1.0 + mant / 8.0, (e - 7).astype(np.int64))
    sub = np.ldexp(mant / 8.0, -6)
    val = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & (mant == 7), np.nan, val)


def dequantise(codes, descale: float):
    """descale * E4M3(codes) in fp64; descale is taken as an fp32 number,
    the precision of the library's descale arguments."""
    return e4m3_value(codes) * float(np.float32(descale))


def attention_fp8(q8, k8, v8, q_descale: float, k_descale: float, v_descale: float, scale: float,
                  causal: bool = False, window: int = 0, rows=None, nthreads=None):
    """Exact attention (dict(o, lse, m, l) as ``oracle.attention``) of the
    dequantised inputs; q8 [B,H,Nq,d], k8, v8 [B,Hkv,Nk,d] are E4M3 codes."""
    return _attention(dequantise(q8, q_descale), dequantise(k8, k_descale), dequantise(v8, v_descale),
                      float(np.float32(scale)), causal, window, rows=rows, nthreads=nthreads)
