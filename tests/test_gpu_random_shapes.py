"""Seeded random shapes for the forward kernels against the oracle: random
batch, head group, query and key lengths (ragged against the 256-row query
tiles and 64-key tiles), head size, causal / window / soft-cap choices.
Tolerances are those of tests/test_gpu_parity.py (bf16, fp32) and
tests/test_gpu_fp8.py (fp8 bounds from E4M3 rounding and the fp8
instruction's accumulation).

FA_RANDOM_SHAPES_SCALE=k multiplies the number of seeds of every family (a
longer sweep: k = 125 runs 1500 bf16, 1500 fp8, 1750 split-KV and 750 fp32
cases in a few minutes on one MI355X)."""
import math
import os

import numpy as np
import pytest

import test_gpu_fp8 as t8
import test_gpu_parity as tp

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
