"""Seeded synthetic inputs for the attention workloads.

This module draws inputs and counts work; it holds none of the attention
arithmetic, so both the GPU path and the CPU oracle can take their inputs
from it.  numpy's PCG64 generator (``numpy.random.default_rng(seed)``)
draws fp32 values in the order Q, K, V; bf16 workloads are then rounded to
bf16 with round-to-nearest-even, and the very same rounded values (exact in
fp32 and fp64) feed both sides.

Workloads (the shapes the pages and the brief describe):

* ``fp32_n64_d32`` -- one head, fp32, 64 queries x 64 keys, d = 32,
  non-causal, scale 1/sqrt(32), uniform[-0.5, 0.5] inputs; the shape of the
  nx_flashattn_scale.nx check (n = 64, d = 32), whose deterministic
  (i*a + dd*b) mod m input pattern is also available as
  :func:`fa_seed_pattern`.
* ``bf16_b1_h8_n1024_d64`` -- non-causal bf16, B=1, H=8, 1024 x 1024, d=64.
* ``bf16_causal_b4_h32_n4096_d128`` -- causal bf16 prefill, B=4, H=32,
  4096 x 4096, d=128 (a Llama-block-shaped attention).
* ``bf16_gqa_swa_softcap_h32kv8_n16384_d128`` -- causal bf16 long-context
  prefill, 32 query heads over 8 key/value heads, 16384 x 16384, d=128,
  a 4096-key sliding window on even query heads and full causal on odd
  ones, logit soft-cap 50.
* ``bf16_splitkv_decode_b16_h32kv8_nk32768_d128`` -- bf16 decode, one query
  per head, B=16, 32 query heads over 8 KV heads, 32768 keys, cut into 16
  splits that are merged afterwards.

fp8 workloads (``FP8_PREFILL``: the causal prefill shape with E4M3 Q, K, V)
draw the same fp32 normals and quantise each tensor with one scale:
descale = max|x| / 448 (E4M3's largest value) and codes = E4M3(x /
descale), round-to-nearest-even (:func:`to_e4m3`).

All tensors are row-major: Q [B,H,Nq,d], K and V [B,Hkv,Nk,d].
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    dtype: str                 # "fp32", "bf16" or "fp8": the tensors' storage type
    causal: bool
    scale: float
    seed: int
    dist: str = "normal"       # "normal": N(0,1); "uniform": U[-0.5, 0.5]
    window: int = 0            # one window for every head (0: none)
    head_window: tuple | None = None  # per query head; overrides window
    softcap: float = 0.0
    num_splits: int = 0        # > 0: split-KV decode with that many splits
    extra: dict = field(default_factory=dict, compare=False)

    def windows(self) -> np.ndarray:
        if self.head_window is not None:
            return np.asarray(self.head_window, dtype=np.int64)
        return np.full(self.H, self.window, dtype=np.int64)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def _even_head_window(H: int, W: int) -> tuple:
    return tuple(W if h % 2 == 0 else 0 for h in range(H))


WORKLOADS = {
    w.name: w for w in [
        Workload("fp32_n64_d32", 1, 1, 1, 64, 64, 32, "fp32", False,
                 1.0 / math.sqrt(32), seed=1, dist="uniform"),
        Workload("bf16_b1_h8_n1024_d64", 1, 8, 8, 1024, 1024, 64, "bf16", False,
                 1.0 / math.sqrt(64), seed=2),
        Workload("bf16_causal_b4_h32_n4096_d128", 4, 32, 32, 4096, 4096, 128, "bf16", True,
                 1.0 / math.sqrt(128), seed=3),
        Workload("bf16_gqa_swa_softcap_h32kv8_n16384_d128", 1, 32, 8, 16384, 16384, 128,
                 "bf16", True, 1.0 / math.sqrt(128), seed=4,
                 head_window=_even_head_window(32, 4096), softcap=50.0),
        Workload("bf16_splitkv_decode_b16_h32kv8_nk32768_d128", 16, 32, 8, 1, 32768, 128,
                 "bf16", False, 1.0 / math.sqrt(128), seed=5, num_splits=16),
    ]
}


# The causal prefill shape with fp8 (E4M3) Q, K, V and bf16 output.
FP8_PREFILL = Workload("fp8_causal_b4_h32_n4096_d128", 4, 32, 32, 4096, 4096, 128, "fp8", True,
                       1.0 / math.sqrt(128), seed=8)


@dataclass(frozen=True)
class RollingWorkload:
    """Streaming decode over a rolling KV cache (Transformers & Math 16.3
    window, 16.6 attention sinks): B sequences, each at position ``pos``,
    one query token per sequence, a cache of ``sinks + window`` rows per
    (sequence, K/V head)."""
    name: str
    B: int
    H: int
    Hkv: int
    d: int
    window: int
    sinks: int
    pos: int
    num_splits: int
    seed: int
    scale: float = 0.0

    @property
    def rows(self) -> int:
        """Filled cache rows: the sink tokens and the window."""
        return min(self.pos + 1, self.sinks + self.window)


# Streaming decode at the pages' window (4096) with 4 sink tokens, on the
# split-KV decode workload's batch and head shape, far into the stream.
ROLLING = RollingWorkload("bf16_rolling_decode_b16_h32kv8_w4096_s4_d128", 16, 32, 8, 128, 4096, 4, 65535, 4,
                          seed=6, scale=1.0 / math.sqrt(128))


def rolling_bytes(w: RollingWorkload) -> int:
    """Bytes one streaming step must move: the new token's K and V read and
    written into the cache, every filled cache row of K and V read once, Q
    read, O and lse written, and the fp32 partials written and read."""
    kv_row = w.B * w.Hkv * w.d * 2
    append = 2 * 2 * kv_row
    cache = 2 * w.rows * kv_row
    q = o = w.B * w.H * w.d * 2
    lse = w.B * w.H * 4
    part = w.B * w.H * w.num_splits * (w.d + 2) * 4
    return append + cache + q + o + lse + 2 * part


@dataclass(frozen=True)
class SoftmaxWorkload:
    """Row softmax over a vocabulary-sized axis: ``rows`` rows of ``n`` fp32
    logits, and the ``k`` largest probabilities of each row."""
    name: str
    rows: int
    n: int
    k: int
    seed: int


# The first Gemma's 256,000-token vocabulary (Transformers & Math 16.3), 512
# rows of logits: 1 MB per row, more than a CU's LDS, so the online
# normaliser's two reads are the minimum for the full softmax.
SOFTMAX = SoftmaxWorkload("fp32_softmax_rows512_n256000", 512, 256000, 8, seed=7)


def softmax_bytes(w: SoftmaxWorkload) -> dict:
    """Bytes each pass structure must move: the online softmax reads x twice
    and writes y once (the safe three-pass softmax reads it three times); the
    fused top-k reads x once and writes k (probability, index) pairs."""
    x = w.rows * w.n * 4
    return {"softmax_online": 2 * x + x + w.rows * 4, "softmax_three_pass": 3 * x + x + w.rows * 4,
            "topk_fused": x + w.rows * w.k * 8 + w.rows * 4}


# The order in which the workloads are listed above; index 0 is the small
# case, index 2 the causal prefill the prefill throughput is quoted on.
ORDER = list(WORKLOADS)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32
    arrays holding exactly representable bf16 values.  Inputs here are
    finite, so NaN handling is not needed."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of fp32 values that are exact bf16 numbers."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("values are not exact bf16 numbers")
    return (u >> 16).astype(np.uint16)


def draw(shape, rng: np.random.Generator, dist: str) -> np.ndarray:
    if dist == "normal":
        return rng.standard_normal(shape, dtype=np.float32)
    if dist == "uniform":
        return rng.random(shape, dtype=np.float32) - np.float32(0.5)
    raise ValueError(dist)


def generate(w: Workload, seed: int | None = None) -> dict:
    """Q, K, V for workload ``w`` as fp32 numpy arrays (bf16-exact values
    for bf16 workloads)."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    q = draw((w.B, w.H, w.Nq, w.d), rng, w.dist)
    k = draw((w.B, w.Hkv, w.Nk, w.d), rng, w.dist)
    v = draw((w.B, w.Hkv, w.Nk, w.d), rng, w.dist)
    if w.dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    return {"q": q, "k": k, "v": v}


def to_e4m3(x: np.ndarray):
    """(codes, descale): x quantised to OCP E4M3 bytes with one fp32 scale,
    descale = max|x| / 448, codes = E4M3(x / descale) rounded to nearest
    (ties to even) by torch's CPU float8_e4m3fn conversion."""
    import torch
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    descale = np.float32(amax / 448.0) if amax > 0 else np.float32(1.0)
    y = np.clip(x / descale, -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return codes, float(descale)


def generate_fp8(w: Workload, seed: int | None = None) -> dict:
    """E4M3 codes (uint8) of Q, K, V drawn as in :func:`generate`, and their
    descale factors: dict(q, k, v, q_descale, k_descale, v_descale)."""
    x = generate(w.with_(dtype="fp32"), seed)
    out = {}
    for n in "qkv":
        out[n], out[n + "_descale"] = to_e4m3(x[n])
    return out


def fa_seed_pattern(n: int, d: int) -> dict:
    """The deterministic input pattern of nx_flashattn_scale.nx (fa_seed):
    x = (i*a + dd*b) mod m mapped to (x - floor(m/2)) / m in fp32, with
    (a, b, m) = (7, 3, 13) for Q, (5, 2, 11) for K and (3, 1, 9) for V."""
    i = np.arange(n, dtype=np.int64)[:, None]
    dd = np.arange(d, dtype=np.int64)[None, :]

    def pat(a, b, m):
        x = (i * a + dd * b) % m
        return (np.float32(x - m // 2) / np.float32(m)).astype(np.float32)

    shape = (1, 1, n, d)
    return {"q": pat(7, 3, 13).reshape(shape), "k": pat(5, 2, 11).reshape(shape),
            "v": pat(3, 1, 9).reshape(shape)}


def worked_example(d: int = 32, dtype=np.float64) -> dict:
    """The notebook's four-key example as attention inputs: one query row
    q = e_0, keys k_i = (1000 + ln i) e_0 for i = 1..4, values v_i = 10 i in
    every column, scale 1.  With dtype float32 the scores are the fp32
    roundings of 1000 + ln i."""
    q = np.zeros((1, 1, 1, d), dtype=dtype)
    q[..., 0] = 1
    k = np.zeros((1, 1, 4, d), dtype=dtype)
    k[0, 0, :, 0] = (1000.0 + np.log(np.arange(1, 5, dtype=np.float64))).astype(dtype)
    v = np.zeros((1, 1, 4, d), dtype=dtype)
    v[0, 0, :, :] = (10.0 * np.arange(1, 5, dtype=np.float64))[:, None].astype(dtype)
    return {"q": q, "k": k, "v": v, "scale": 1.0}


def visible_counts(w: Workload) -> np.ndarray:
    """Number of visible keys of every query row, per head: [H, Nq]."""
    i = np.arange(w.Nq, dtype=np.int64)
    p = i + (w.Nk - w.Nq)
    out = np.empty((w.H, w.Nq), dtype=np.int64)
    for h, W in enumerate(w.windows()):
        hi = np.minimum(p + 1, w.Nk) if w.causal else np.full_like(p, w.Nk)
        lo = np.maximum(p - W + 1, 0) if W > 0 else np.zeros_like(p)
        out[h] = np.maximum(hi - lo, 0)
    return out


def algorithmic_flops(w: Workload) -> int:
    """2d FLOPs for Q.K and 2d for P.V per (query, visible key) pair."""
    pairs = int(visible_counts(w).sum()) * w.B
    return 4 * w.d * pairs


def algorithmic_bytes(w: Workload) -> int:
    """Bytes a perfect kernel must move through HBM: Q, K and V read once,
    O and the fp32 row lse written once; split-KV also writes and reads its
    fp32 partials (O_s, m_s, l_s)."""
    es = {"fp32": 4, "bf16": 2, "fp8": 1}[w.dtype]
    q = w.B * w.H * w.Nq * w.d * es
    kv = 2 * w.B * w.Hkv * w.Nk * w.d * es
    o = w.B * w.H * w.Nq * w.d * (2 if w.dtype == "fp8" else es)  # fp8 attention writes bf16
    lse = w.B * w.H * w.Nq * 4
    total = q + kv + o + lse
    if w.num_splits:
        part = w.B * w.H * w.Nq * w.num_splits * (w.d + 2) * 4
        total += 2 * part
    return total
