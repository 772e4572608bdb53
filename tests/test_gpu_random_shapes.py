"""Seeded random shapes for the forward kernels against the oracle: random
batch, head group, query and key lengths (ragged against the 256-row query
tiles and 64-key tiles), head size, causal / window / soft-cap choices.
Tolerances are those of tests/test_gpu_parity.py (bf16, fp32) and
tests/test_gpu_fp8.py (fp8 bounds from E4M3 rounding and the fp8
instruction's accumulation).

Also: token streams through a rolling KV cache (random window, sinks, chunk
sizes and check positions) and row softmax / fused top-k over random row
lengths, both with the tolerances of their own test files.

Also: causal bf16 grids with B*Hkv a multiple of 8 and several K/V heads
per XCD, which the block order takes in clusters.

FA_RANDOM_SHAPES_SCALE=k multiplies the number of seeds of every family (a
longer sweep: k = 125 runs 1500 bf16, 1500 fp8, 1750 split-KV and 750 fp32
cases in a few minutes on one MI355X)."""
import math
import os

import numpy as np
import pytest

import test_gpu_fp8 as t8
import test_gpu_parity as tp
import test_gpu_rolling as tr
import test_gpu_softmax as tsm

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

SCALE = max(1, int(os.environ.get("FA_RANDOM_SHAPES_SCALE", "1")))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import online_softmax_tiled_amd as fa
    fa.load_library()
    yield


def draw_shape(rng, ds):
    Hkv = int(rng.choice([1, 2, 4]))
    H = Hkv * int(rng.choice([1, 2, 3, 4]))
    B = int(rng.integers(1, 3))
    Nk = int(rng.integers(1, 700))
    u = rng.random()
    Nq = 1 if u < 0.2 else (int(rng.integers(1, 600)) if u < 0.6 else Nk)
    d = int(rng.choice(ds))
    causal = rng.random() < 0.6
    window = int(rng.integers(1, 300)) if causal and rng.random() < 0.5 else 0
    return B, H, Hkv, Nq, Nk, d, causal, window


@pytest.mark.parametrize("seed", range(12 * SCALE))
def test_bf16_random_shapes(seed):
    rng = np.random.default_rng(1000 + seed)
    B, H, Hkv, Nq, Nk, d, causal, window = draw_shape(rng, [32, 64, 128])
    softcap = float(rng.choice([0.0, 0.0, 20.0]))
    what = f"bf16 seed={seed} B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} W={window} cap={softcap}"
    print("case", what, flush=True)
    inp = tp.rand_inputs(B, H, Hkv, Nq, Nk, d, seed=seed, dtype="bf16")
    tp.parity(inp, "bf16", 1.0 / math.sqrt(d), causal=causal, window=window, softcap=softcap, what=what)


@pytest.mark.parametrize("seed", range(6 * SCALE))
def test_bf16_random_causal_head_clusters(seed):
    # B*Hkv a multiple of 8 with several K/V heads per XCD: the causal block
    # order takes them in clusters (and a short last cluster); both the
    # 8-wave and the 4-wave grids occur.
    rng = np.random.default_rng(7000 + seed)
    Hkv = 8
    H = Hkv * int(rng.choice([1, 2]))
    B = int(rng.integers(3, 7))
    N = int(rng.integers(200, 1100))
    d = int(rng.choice([32, 64]))
    window = int(rng.integers(1, 400)) if rng.random() < 0.3 else 0
    what = f"bf16 clusters seed={seed} B={B} H={H} Hkv={Hkv} N={N} d={d} W={window}"
    print("case", what, flush=True)
    inp = tp.rand_inputs(B, H, Hkv, N, N, d, seed=seed, dtype="bf16")
    tp.parity(inp, "bf16", 1.0 / math.sqrt(d), causal=True, window=window, what=what)


@pytest.mark.parametrize("seed", range(6 * SCALE))
def test_fp32_random_shapes(seed):
    rng = np.random.default_rng(2000 + seed)
    B, H, Hkv, Nq, Nk, d, causal, window = draw_shape(rng, [32, 64, 128])
    what = f"fp32 seed={seed} B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} W={window}"
    print("case", what, flush=True)
    inp = tp.rand_inputs(B, H, Hkv, Nq, Nk, d, seed=seed, dtype="fp32", dist="uniform")
    tp.parity(inp, "fp32", 1.0 / math.sqrt(d), causal=causal, window=window, what=what)


@pytest.mark.parametrize("seed", range(10 * SCALE))
def test_fp8_random_shapes(seed):
    rng = np.random.default_rng(3000 + seed)
    B, H, Hkv, Nq, Nk, d, causal, window = draw_shape(rng, [64, 128])
    family = ("narrow", "full range")[seed % 2]
    what = (f"fp8 {family} seed={seed} B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} "
            f"W={window}")
    print("case", what, flush=True)
    make = t8.narrow_inputs if family == "narrow" else t8.random_inputs
    t8.check(make(B, H, Hkv, Nq, Nk, d, seed=seed), 1.0 / math.sqrt(d), causal, window, what)


@pytest.mark.parametrize("seed", range(14 * SCALE))
def test_splitkv_random_shapes(seed):
    # Few rows per K/V head take the decode kernel (1, 2 or 4 rows per
    # pass), more take the MFMA kernel in split mode; up to 16 splits and
    # more take different combine kernels.
    rng = np.random.default_rng(4000 + seed)
    Hkv = int(rng.choice([1, 2, 4]))
    H = Hkv * int(rng.choice([1, 2, 4, 8]))
    B = int(rng.integers(1, 3))
    Nk = int(rng.integers(1, 3000))
    Nq = int(rng.choice([1, 1, 2, int(rng.integers(3, 70))]))
    d = int(rng.choice([32, 64, 128]))
    S = int(rng.choice([1, 2, 5, 16, 17, 40]))
    causal = rng.random() < 0.5
    window = int(rng.integers(1, 400)) if causal and rng.random() < 0.5 else 0
    softcap = float(rng.choice([0.0, 0.0, 30.0]))
    scale = 1.0 / math.sqrt(d)
    what = (f"split seed={seed} B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} S={S} causal={causal} W={window} "
            f"cap={softcap}")
    print("case", what, flush=True)
    inp = tp.rand_inputs(B, H, Hkv, Nq, Nk, d, seed=seed, dtype="bf16")
    kw = dict(causal=causal, window=window, softcap=softcap)
    o, lse, (op, mp, lp) = tp.run_split(inp, S, scale, **kw)
    ref = tp.oracle.attention(inp["q"], inp["k"], inp["v"], scale, **kw)
    tp.check_o(o, ref["o"], "bf16", what)
    tp.check_lse(lse, ref["lse"], "bf16", what)
    rop, rmp, rlp = tp.oracle.split_partials(inp["q"], inp["k"], inp["v"], scale, S, **kw)
    fin = np.isfinite(rmp)
    assert np.array_equal(fin, np.isfinite(mp)), what
    assert np.all(lp[~fin] == 0) and np.all(op[~fin] == 0), what
    assert np.allclose(mp[fin], rmp[fin], rtol=1e-3, atol=1e-3), what
    assert np.allclose(lp[fin], rlp[fin], rtol=tp.BF16_LSE, atol=0), what
    assert np.max(np.abs(op - rop), initial=0.0) < tp.BF16_MAX, what


@pytest.mark.parametrize("seed", range(8 * SCALE))
def test_rolling_random_streams(seed):
    rng = np.random.default_rng(5000 + seed)
    Hkv = int(rng.choice([1, 2, 4]))
    H = Hkv * int(rng.choice([1, 2, 4, 16]))
    B = int(rng.integers(1, 3))
    d = int(rng.choice([32, 64, 128]))
    W = int(rng.integers(1, 200))
    S = int(rng.choice([0, 1, 4]))
    nsplit = int(rng.choice([1, 2, 3, 5, 17]))
    cap = float(rng.choice([0.0, 0.0, 30.0]))
    N = int(rng.integers(1, 500))
    pre = int(rng.integers(1, N + 1))
    checks = sorted(set([pre - 1, N - 1] + [int(x) for x in rng.integers(pre - 1, N, 3)]))
    what = f"rolling seed={seed} B={B} H={H} Hkv={Hkv} d={d} W={W} sinks={S} N={N} pre={pre} S={nsplit} cap={cap}"
    print("case", what, flush=True)
    inp = tr.seq_inputs(B, H, Hkv, N, d, seed=seed)
    k_all, v_all = tr.dev(inp["k"]), tr.dev(inp["v"])
    cache = tr.fa_mod().RollingKVCache(B, Hkv, d, W, S)
    scale = 1.0 / math.sqrt(d)
    pos = -1
    while pos < checks[-1]:
        T = pre if pos < 0 else int(rng.integers(1, 4))
        T = min(T, N - 1 - pos)
        cache.append(k_all[:, :, pos + 1:pos + 1 + T].contiguous(), v_all[:, :, pos + 1:pos + 1 + T].contiguous())
        pos += T
        if pos in checks:
            tr.check_decode(cache, inp, pos, W, S, scale, cap, nsplit, f"{what} pos={pos}")
    torch.cuda.synchronize()
    tr.check_cache(cache, inp["k"], inp["v"], pos, W, S)


@pytest.mark.parametrize("seed", range(8 * SCALE))
def test_softmax_random_rows(seed):
    rng = np.random.default_rng(6000 + seed)
    dtype = str(rng.choice(["fp32", "bf16"]))
    rows = int(rng.integers(1, 9))
    n = int(rng.choice([int(rng.integers(1, 300)), int(rng.integers(300, 40000)), int(rng.integers(40000, 300000))]))
    scale = float(rng.choice([1e-3, 1.0, 3.0, 30.0]))
    shift = float(rng.choice([0.0, -200.0, 500.0]))
    k = int(rng.integers(1, min(64, n) + 1))
    what = f"softmax seed={seed} {dtype} rows={rows} n={n} scale={scale} shift={shift} k={k}"
    print("case", what, flush=True)
    x = tsm.logits(rows, n, seed=seed, dtype=dtype, scale=scale, shift=shift)
    tsm.check_softmax(x, dtype, what)
    tsm.check_topk(x, dtype, k, what)
