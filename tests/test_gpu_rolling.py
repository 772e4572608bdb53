"""Rolling KV cache with attention sinks (fa_kv_append, fa_decode_rolling +
fa_combine) against the fp64 oracle.

A stream of tokens is written into the cache (a chunk, then one token at a
time); at chosen positions the decode query attends to the cache and must
match the oracle's attention over the whole sequence with the causal rule,
a window of the last W positions and the first `sinks` tokens kept
(Transformers & Math 16.3 and 16.6).  The cache contents are byte copies
and are compared exactly with the ring rule.  bf16 tolerances as in
test_gpu_parity.
"""
import math

import numpy as np
import pytest

import oracle
from online_softmax_tiled_amd import workloads as wl

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN = 2e-2, 2e-3
BF16_LSE = 1e-4  # lse relative bound (the normaliser sums fp32 weights)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import online_softmax_tiled_amd as fa
    fa.load_library()
    yield


def fa_mod():
    import online_softmax_tiled_amd as fa
    return fa


def seq_inputs(B, H, Hkv, N, d, seed):
    w = wl.Workload("rolling", B, H, Hkv, N, N, d, "bf16", True, 1.0, seed)
    return wl.generate(w)


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).cuda()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def ring_row(t, window, sinks):
    return t if t < sinks else sinks + (t - sinks) % window


def check_cache(cache, k, v, pos, window, sinks):
    """After tokens 0..pos: every filled row holds exactly the latest token
    mapped to it (bit-exact bf16 copy)."""
    kc, vc = host(cache.k), host(cache.v)
    latest = {}
    for t in range(pos + 1):
        latest[ring_row(t, window, sinks)] = t
    rows = sorted(latest)
    assert rows == list(range(len(rows)))
    idx = [latest[r] for r in rows]
    assert np.array_equal(kc[:, :, :len(rows)], k[:, :, idx].astype(np.float64))
    assert np.array_equal(vc[:, :, :len(rows)], v[:, :, idx].astype(np.float64))


def check_decode(cache, inp, pos, window, sinks, scale, softcap, S, what):
    q = dev(inp["q"][:, :, pos:pos + 1])
    o, lse = cache.attend(q, num_splits=S, scale=scale, softcap=softcap)
    torch.cuda.synchronize()
    ref = oracle.attention(inp["q"][:, :, pos:pos + 1], inp["k"][:, :, :pos + 1], inp["v"][:, :, :pos + 1],
                           scale, causal=True, window=window, softcap=softcap, sinks=sinks)
    err = np.abs(host(o) - ref["o"])
    assert np.all(np.isfinite(host(o))), what
    assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN, f"{what}: err max {err.max():.3g} mean {err.mean():.3g}"
    lerr = np.abs(host(lse) - ref["lse"]) / np.maximum(1.0, np.abs(ref["lse"]))
    assert lerr.max() <= BF16_LSE, f"{what}: lse rel err {lerr.max():.3g}"


# B, H, Hkv, d, window, sinks, prefill chunk, positions checked, num_splits, softcap
CASES = [
    (2, 8, 2, 128, 64, 4, 40, [1, 3, 39, 60, 67, 68, 200, 333], 4, 0.0),
    (1, 4, 4, 64, 32, 4, 100, [100, 101, 129, 257], 3, 0.0),
    (2, 32, 2, 128, 48, 4, 20, [20, 51, 52, 140], 5, 0.0),   # 16 query heads per K/V head: MFMA split path
    (1, 8, 1, 32, 16, 0, 10, [10, 15, 16, 75], 2, 0.0),        # no sinks: a plain ring of the window
    (1, 8, 2, 128, 64, 4, 70, [70, 150], 8, 30.0),           # soft-capped scores
]


@pytest.mark.parametrize("n", range(len(CASES)))
def test_rolling_decode_stream(n):
    B, H, Hkv, d, W, S, pre, checks, nsplit, cap = CASES[n]
    N = max(checks) + 1
    print(f"case rolling n={n} B={B} H={H} Hkv={Hkv} d={d} W={W} sinks={S} N={N}", flush=True)
    inp = seq_inputs(B, H, Hkv, N, d, seed=60 + n)
    k_all, v_all = dev(inp["k"]), dev(inp["v"])
    cache = fa_mod().RollingKVCache(B, Hkv, d, W, S)
    scale = 1.0 / math.sqrt(d)
    pos = -1
    targets = sorted(set(checks))
    while pos < targets[-1]:
        T = pre if pos < 0 else 1
        if pos < 0 and T - 1 > targets[0]:
            T = targets[0] + 1
        cache.append(k_all[:, :, pos + 1:pos + 1 + T].contiguous(), v_all[:, :, pos + 1:pos + 1 + T].contiguous())
        pos += T
        if pos in targets:
            check_decode(cache, inp, pos, W, S, scale, cap, nsplit, f"rolling n={n} pos={pos}")
    torch.cuda.synchronize()
    check_cache(cache, inp["k"], inp["v"], pos, W, S)


@pytest.mark.parametrize("T", [1, 37, 64, 65, 150])
def test_append_chunk_replaces_like_single_tokens(T):
    # a chunk longer than the window keeps only its last tokens in the ring
    B, Hkv, d, W, S = 2, 3, 64, 32, 4
    start = 5
    print(f"case append T={T}", flush=True)
    inp = seq_inputs(B, Hkv, Hkv, start + T, d, seed=90 + T)
    k_all, v_all = dev(inp["k"]), dev(inp["v"])
    cache = fa_mod().RollingKVCache(B, Hkv, d, W, S)
    cache.append(k_all[:, :, :start].contiguous(), v_all[:, :, :start].contiguous())
    cache.append(k_all[:, :, start:].contiguous(), v_all[:, :, start:].contiguous())
    torch.cuda.synchronize()
    check_cache(cache, inp["k"], inp["v"], start + T - 1, W, S)


def test_rolling_bench_shape_sampled():
    # the benchmark's configuration: B=16, H=32, Hkv=8, d=128, W=4096,
    # sinks=4, position 65535 (the ring has wrapped many times), 4 splits.
    # The cache is filled directly in ring order from a synthetic sequence
    # of its own rows; a few batches are checked against the oracle.
    B, H, Hkv, d, W, S = 16, 32, 8, 128, 4096, 4
    pos = 65535
    print("case rolling bench shape", flush=True)
    rng = np.random.default_rng(7)
    rows = S + W
    kc = wl.round_bf16(rng.standard_normal((B, Hkv, rows, d)).astype(np.float32))
    vc = wl.round_bf16(rng.standard_normal((B, Hkv, rows, d)).astype(np.float32))
    q = wl.round_bf16(rng.standard_normal((B, H, 1, d)).astype(np.float32))
    fa = fa_mod()
    cache = fa.RollingKVCache(B, Hkv, d, W, S)
    cache.k.copy_(dev(kc))
    cache.v.copy_(dev(vc))
    cache.length = pos + 1
    o, lse = cache.attend(dev(q), num_splits=4)
    torch.cuda.synchronize()
    # every filled row is visible: plain attention over the cache rows
    for b in (0, 9, 15):
        ref = oracle.attention(q[b:b + 1], kc[b:b + 1], vc[b:b + 1], 1.0 / math.sqrt(d))
        err = np.abs(host(o)[b:b + 1] - ref["o"])
        assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN
        assert np.allclose(host(lse)[b:b + 1], ref["lse"], rtol=BF16_LSE, atol=BF16_LSE)
