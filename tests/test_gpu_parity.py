"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle.

Inputs come from the seeded generators in online_softmax_tiled_amd.workloads;
the same bf16/fp32 values go to both sides.  Tolerances:
  * fp32 paths: max |O_gpu - O_oracle| <= 1e-5, |lse| error <= 1e-5 * max(1, |lse|);
  * bf16 paths: max abs error <= 2e-2 and mean abs error <= 2e-3 on O,
    |lse| error <= 1e-4 * max(1, |lse|) (every bf16 path sums the fp32 weights
    into the normaliser, so lse carries no bf16 rounding; the partial sums
    are held to the same relative bound).
Full-size workloads are checked on every row, in the launch configuration
the benchmark times.
"""
import math

import numpy as np
import pytest

import oracle
from online_softmax_tiled_amd import workloads as wl

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

FP32_TOL = 1e-5
BF16_MAX, BF16_MEAN = 2e-2, 2e-3
BF16_LSE = 1e-4


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


def dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(dtype).cuda()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def check_o(o_gpu, o_ref, dtype, what=""):
    err = np.abs(o_gpu - o_ref)
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite output"
    if dtype == "fp32":
        assert err.max() <= FP32_TOL, f"{what}: max abs err {err.max():.3g}"
    else:
        assert err.max() <= BF16_MAX, f"{what}: max abs err {err.max():.3g}"
        assert err.mean() <= BF16_MEAN, f"{what}: mean abs err {err.mean():.3g}"


def check_lse(lse_gpu, lse_ref, dtype, what=""):
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(lse_gpu)), f"{what}: -inf pattern differs"
    assert np.all(lse_gpu[~fin] == -np.inf)
    rel = (FP32_TOL if dtype == "fp32" else BF16_LSE)
    err = np.abs(lse_gpu[fin] - lse_ref[fin]) / np.maximum(1.0, np.abs(lse_ref[fin]))
    assert err.size == 0 or err.max() <= rel, f"{what}: lse rel err {err.max():.3g}"


def run_gpu(inp, dtype, scale, causal=False, window=0, head_window=None, softcap=0.0):
    tdt = torch.float32 if dtype == "fp32" else torch.bfloat16
    q, k, v = dev(inp["q"], tdt), dev(inp["k"], tdt), dev(inp["v"], tdt)
    # Outputs start as NaN: an element the kernel does not write fails.
    o = torch.full(q.shape, float("nan"), dtype=tdt, device="cuda")
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    o, lse = fa_mod().attention(q, k, v, scale=scale, causal=causal, window=window,
                                head_window=head_window, softcap=softcap, out=o, lse=lse)
    torch.cuda.synchronize()
    return host(o), host(lse)


def parity(inp, dtype, scale, causal=False, window=0, head_window=None, softcap=0.0, what=""):
    o, lse = run_gpu(inp, dtype, scale, causal, window, head_window, softcap)
    ref = oracle.attention(inp["q"], inp["k"], inp["v"], scale, causal=causal, window=window,
                           head_window=head_window, softcap=softcap)
    check_o(o, ref["o"], dtype, what)
    check_lse(lse, ref["lse"], dtype, what)
    return o, lse, ref


def rand_inputs(B, H, Hkv, Nq, Nk, d, seed, dtype, scale_in=1.0, dist="normal"):
    w = wl.Workload("t", B, H, Hkv, Nq, Nk, d, dtype, False, 1.0, seed, dist=dist)
    inp = wl.generate(w)
    if scale_in != 1.0:
        inp = {n: (x * np.float32(scale_in)) for n, x in inp.items()}
        if dtype == "bf16":
            inp = {n: wl.round_bf16(x) for n, x in inp.items()}
    return inp


# ----------------------------------------------------------------- fp32 path
def test_fp32_workload_full():
    w = wl.WORKLOADS["fp32_n64_d32"]
    print(f"case {w.name}", flush=True)
    parity(wl.generate(w), "fp32", w.scale, what=w.name)


def test_fp32_worked_example():
    we = wl.worked_example(d=32, dtype=np.float32)
    o, lse, ref = parity(we, "fp32", 1.0, what="worked example")
    # fp32 scores are the roundings of 1000 + ln i; their exact softmax is
    # 29.99993039..., and 30.0 within the rounding of the inputs.
    assert abs(o[0, 0, 0, 0] - 29.99993039) < 1e-5
    assert abs(o[0, 0, 0, 0] - 30.0) < 1e-4


def test_fp32_fa_seed_pattern():
    p = wl.fa_seed_pattern(64, 32)
    parity(p, "fp32", 1.0 / math.sqrt(32), what="fa_seed pattern")


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("mode", ["plain", "causal", "window", "softcap", "gqa_cross"])
def test_fp32_shapes(d, mode):
    B, H, Hkv, Nq, Nk = 2, 4, 4, 77, 133
    kw = {}
    if mode == "causal":
        kw = dict(causal=True)
    elif mode == "window":
        kw = dict(causal=True, head_window=[0, 5, 40, 1])
    elif mode == "softcap":
        kw = dict(causal=True, softcap=2.0)
    elif mode == "gqa_cross":
        Hkv, Nq, Nk = 2, 5, 200
    inp = rand_inputs(B, H, Hkv, Nq, Nk, d, seed=31 + d, dtype="fp32", dist="uniform")
    parity(inp, "fp32", 1.0 / math.sqrt(d) * 3, what=f"fp32 {mode} d={d}", **kw)


# ----------------------------------------------------------------- bf16 path
def test_bf16_workload_full():
    w = wl.WORKLOADS["bf16_b1_h8_n1024_d64"]
    print(f"case {w.name}", flush=True)
    parity(wl.generate(w), "bf16", w.scale, what=w.name)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("mode", ["plain", "causal", "window", "softcap", "gqa", "cross"])
def test_bf16_shapes(d, mode):
    # several 128-row query tiles and 64-key tiles, with ragged tails
    B, H, Hkv, Nq, Nk = 2, 4, 4, 300, 333
    kw = {}
    if mode == "causal":
        kw = dict(causal=True)
    elif mode == "window":
        kw = dict(causal=True, head_window=[0, 64, 100, 7])
    elif mode == "softcap":
        kw = dict(causal=True, softcap=5.0)
    elif mode == "gqa":
        Hkv = 1
        kw = dict(causal=True, window=90)
    elif mode == "cross":
        Nq, Nk = 130, 700
    print(f"case bf16 {mode} d={d}", flush=True)
    inp = rand_inputs(B, H, Hkv, Nq, Nk, d, seed=7 + d, dtype="bf16")
    parity(inp, "bf16", 1.0 / math.sqrt(d), what=f"bf16 {mode} d={d}", **kw)


@pytest.mark.parametrize("shape", [(5, 32, 8, 1024, 64, 0), (5, 32, 8, 1024, 128, 300), (7, 8, 8, 4096, 32, 0)])
def test_bf16_causal_block_order_clusters(shape):
    # Causal grids whose B*Hkv is a multiple of 8 take their K/V heads in
    # clusters per XCD; these shapes give clusters of 4 + 1 and 4 + 3 heads
    # per XCD (a short last cluster).  Every row must be written once.
    B, H, Hkv, N, d, W = shape
    print(f"case bf16 block order {shape}", flush=True)
    inp = rand_inputs(B, H, Hkv, N, N, d, seed=B * N + d, dtype="bf16")
    parity(inp, "bf16", 1.0 / math.sqrt(d), causal=True, window=W, what=f"bf16 block order {shape}")


def test_bf16_large_scores_stay_finite():
    # Scores scaled by 40: without the running maximum they overflow.
    inp = rand_inputs(1, 2, 2, 200, 260, 64, seed=5, dtype="bf16")
    parity(inp, "bf16", 40.0 / math.sqrt(64), causal=True, what="bf16 x40")


def test_fp32_large_scores_stay_finite():
    # The fp32 workload's inputs (uniform[-0.5, 0.5], d = 32) with scores
    # multiplied by 40.  The 1e-5 bar holds for scores of this size; it is
    # not a bound for arbitrary magnitudes (fp32 rounding of a score s alone
    # is ~|s| * 6e-8).
    inp = rand_inputs(1, 2, 2, 70, 90, 32, seed=6, dtype="fp32", dist="uniform")
    parity(inp, "fp32", 40.0 / math.sqrt(32), what="fp32 x40")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_empty_and_masked_rows(dtype):
    # Nk = 0: every row sees nothing -> O = 0, lse = -inf.
    inp = rand_inputs(1, 2, 2, 9, 0, 64, seed=8, dtype=dtype)
    o, lse = run_gpu(inp, dtype, 0.125)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    # More queries than keys under a causal mask: the first rows see no key.
    inp = rand_inputs(1, 2, 2, 150, 20, 64, seed=9, dtype=dtype)
    o, lse, ref = parity(inp, dtype, 0.125, causal=True, what="causal Nq > Nk")
    assert np.all(o[:, :, :130] == 0) and np.all(np.isneginf(lse[:, :, :130]))
    # Nq = 0 is a no-op.
    inp = rand_inputs(1, 2, 2, 0, 20, 64, seed=10, dtype=dtype)
    o, lse = run_gpu(inp, dtype, 0.125)
    assert o.shape == (1, 2, 0, 64)


def test_single_key_and_uniform_scores():
    rng = np.random.default_rng(11)
    v = wl.round_bf16(rng.standard_normal((1, 2, 1, 128), dtype=np.float32))
    k = wl.round_bf16(rng.standard_normal((1, 2, 1, 128), dtype=np.float32))
    q = wl.round_bf16(rng.standard_normal((1, 2, 5, 128), dtype=np.float32))
    o, lse = run_gpu({"q": q, "k": k, "v": v}, "bf16", 0.1)
    # bf16 output of V exactly (V is bf16 already, weight exactly 1)
    assert np.array_equal(o, np.broadcast_to(v, o.shape).astype(np.float64))
    # q = 0: O is the mean of the visible values, lse = ln(count)
    q0 = np.zeros((1, 2, 70, 64), dtype=np.float32)
    kv = {n: wl.round_bf16(rng.standard_normal((1, 2, 70, 64), dtype=np.float32)) for n in "kv"}
    o, lse = run_gpu({"q": q0, **kv}, "bf16", 1.0, causal=True)
    cnt = np.arange(1, 71)
    assert np.allclose(lse[0, 0], np.log(cnt), atol=1e-5)
    mean = np.cumsum(kv["v"][0].astype(np.float64), axis=1) / cnt[None, :, None]
    assert np.max(np.abs(o[0] - mean)) < 2e-2


# ------------------------------------------------------- full-size, all rows
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["bf16_causal_b4_h32_n4096_d128", "bf16_gqa_swa_softcap_h32kv8_n16384_d128"])
def test_full_size_prefill_all_rows(name):
    # The benchmark's launch at full size, every one of the B*H*Nq rows
    # compared with the oracle (threaded over the host cores), and the
    # max-abs / mean-abs / lse criteria evaluated over the whole output.
    w = wl.WORKLOADS[name]
    print(f"case {name} (full size, all rows)", flush=True)
    inp = wl.generate(w)
    hw = list(w.head_window) if w.head_window else None
    o, lse = run_gpu(inp, "bf16", w.scale, causal=w.causal, window=w.window, head_window=hw,
                     softcap=w.softcap)
    ref = oracle.attention(inp["q"], inp["k"], inp["v"], w.scale, causal=w.causal, window=w.window,
                           head_window=hw, softcap=w.softcap)
    err = np.abs(o - ref["o"])
    lerr = np.abs(lse - ref["lse"]) / np.maximum(1.0, np.abs(ref["lse"]))
    print(f"{name}: all {o.shape[0] * o.shape[1] * o.shape[2]} rows: max |dO| {err.max():.3e}, "
          f"mean |dO| {err.mean():.3e}, max lse rel err {lerr.max():.3e}", flush=True)
    check_o(o, ref["o"], "bf16", name)
    check_lse(lse, ref["lse"], "bf16", name)


# -------------------------------------------------------------- split-KV
def run_split(inp, S, scale, causal=False, window=0, softcap=0.0, out_dtype=None):
    q, k, v = (dev(inp[n], torch.bfloat16) for n in "qkv")
    B, H, Nq, d = q.shape
    # Partials start as NaN: every split of every row must be written
    # (an empty split as m = -inf, l = 0, O = 0).
    nan = float("nan")
    parts = (torch.full((B, H, Nq, S, d), nan, device="cuda"), torch.full((B, H, Nq, S), nan, device="cuda"),
             torch.full((B, H, Nq, S), nan, device="cuda"))
    o, lse, parts = fa_mod().splitkv_attention(q, k, v, S, scale=scale, causal=causal, window=window,
                                               softcap=softcap, out_dtype=out_dtype, partials=parts,
                                               return_partials=True)
    torch.cuda.synchronize()
    return host(o), host(lse), tuple(host(t) for t in parts)


def test_splitkv_decode_workload_full():
    w = wl.WORKLOADS["bf16_splitkv_decode_b16_h32kv8_nk32768_d128"]
    print(f"case {w.name}", flush=True)
    inp = wl.generate(w)
    o, lse, (op, mp, lp) = run_split(inp, w.num_splits, w.scale)
    ref = oracle.attention(inp["q"], inp["k"], inp["v"], w.scale)
    check_o(o, ref["o"], "bf16", w.name)
    check_lse(lse, ref["lse"], "bf16", w.name)
    # The partials are each split's own attention (checked on a few rows).
    rows = np.array([0, 5, 100, 511])
    chunk = -(-w.Nk // w.num_splits)
    for s in (0, 7, 15):
        r = oracle.attention(inp["q"], inp["k"], inp["v"], w.scale, rows=rows,
                             key_range=(s * chunk, min(w.Nk, (s + 1) * chunk)))
        assert np.max(np.abs(op.reshape(-1, w.num_splits, w.d)[rows, s] - r["o"])) < BF16_MAX
        assert np.allclose(mp.reshape(-1, w.num_splits)[rows, s], r["m"], rtol=1e-3, atol=1e-3)
        assert np.allclose(lp.reshape(-1, w.num_splits)[rows, s], r["l"], rtol=BF16_LSE)


@pytest.mark.parametrize("S", [1, 2, 3, 16, 17, 40])  # <= 16 and > 16 take different combine kernels
@pytest.mark.parametrize("shape", [(2, 8, 2, 1, 1000, 128), (1, 4, 4, 2, 517, 64), (2, 8, 1, 1, 300, 32),
                                   (1, 4, 2, 40, 700, 128)])
def test_splitkv_matches_unsplit(S, shape):
    B, H, Hkv, Nq, Nk, d = shape
    print(f"case splitkv S={S} shape={shape}", flush=True)
    inp = rand_inputs(B, H, Hkv, Nq, Nk, d, seed=20 + S, dtype="bf16")
    kw = dict(causal=True, softcap=30.0) if Nq > 1 else {}
    o, lse, (op, mp, lp) = run_split(inp, S, 1.0 / math.sqrt(d), **kw)
    ref = oracle.attention(inp["q"], inp["k"], inp["v"], 1.0 / math.sqrt(d), **kw)
    check_o(o, ref["o"], "bf16", f"split S={S}")
    check_lse(lse, ref["lse"], "bf16", f"split S={S}")
    # Each partial is its chunk's own (maximum, sum, normalised output).
    rop, rmp, rlp = oracle.split_partials(inp["q"], inp["k"], inp["v"], 1.0 / math.sqrt(d), S, **kw)
    fin = np.isfinite(rmp)
    assert np.array_equal(fin, np.isfinite(mp)) and np.all(lp[~fin] == 0)
    assert np.allclose(mp[fin], rmp[fin], rtol=1e-3, atol=1e-3)
    assert np.allclose(lp[fin], rlp[fin], rtol=BF16_LSE, atol=0)
    assert np.max(np.abs(op - rop)) < BF16_MAX


def test_splitkv_mfma_rows_outside_a_split():
    # Enough query rows per K/V head for the MFMA kernel in split mode; with
    # a 100-key causal window most splits hold no key of a given row (on
    # either side of its window), which must give (m, l, O) = (-inf, 0, 0).
    inp = rand_inputs(1, 4, 1, 64, 2048, 128, seed=33, dtype="bf16")
    o, lse, (op, mp, lp) = run_split(inp, 8, 1.0 / math.sqrt(128), causal=True, window=100)
    ref = oracle.attention(inp["q"], inp["k"], inp["v"], 1.0 / math.sqrt(128), causal=True, window=100)
    check_o(o, ref["o"], "bf16", "mfma split, window")
    check_lse(lse, ref["lse"], "bf16", "mfma split, window")
    rop, rmp, rlp = oracle.split_partials(inp["q"], inp["k"], inp["v"], 1.0 / math.sqrt(128), 8, causal=True,
                                          window=100)
    fin = np.isfinite(rmp)
    assert (~fin).sum() > 0 and np.array_equal(fin, np.isfinite(mp))
    assert np.all(lp[~fin] == 0) and np.all(op[~fin] == 0)
    assert np.allclose(lp[fin], rlp[fin], rtol=BF16_LSE, atol=0)


def test_splitkv_window_and_empty_splits():
    # A window leaves most splits empty for the decode row; empty partials
    # must carry no weight.
    inp = rand_inputs(1, 4, 1, 1, 640, 64, seed=30, dtype="bf16")
    o, lse, (op, mp, lp) = run_split(inp, 8, 0.125, causal=True, window=50)
    ref = oracle.attention(inp["q"], inp["k"], inp["v"], 0.125, causal=True, window=50)
    check_o(o, ref["o"], "bf16", "split window")
    check_lse(lse, ref["lse"], "bf16", "split window")
    assert np.all(lp[..., :7] == 0) and np.all(np.isneginf(mp[..., :7]))
    # fp32 output of the combine
    o32, lse32, _ = run_split(inp, 8, 0.125, causal=True, window=50, out_dtype=torch.float32)
    assert np.max(np.abs(o32 - ref["o"])) < 5e-3


def test_combine_merge_exercise_on_gpu():
    # Hand-built partials: block 1 (m=2, l=3), block 2 (m=5, l=1.5); the
    # merged normaliser relative to m=5 is 3e^-3 + 1.5 = 1.6494.
    d = 64
    op = torch.zeros((1, 1, 1, 2, d), dtype=torch.float32)
    op[0, 0, 0, 0, :] = 1.0
    op[0, 0, 0, 1, :] = -1.0
    mp = torch.tensor([[[[2.0, 5.0]]]])
    lp = torch.tensor([[[[3.0, 1.5]]]])
    o = torch.empty((1, 1, 1, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((1, 1, 1), dtype=torch.float32, device="cuda")
    fa = fa_mod()
    fa.fa_combine(op.cuda(), mp.cuda(), lp.cuda(), o, lse, 1, 1, 1, d, 2, 1)
    torch.cuda.synchronize()
    ell = math.exp(float(lse.cpu()[0, 0, 0]) - 5.0)
    assert abs(ell - 1.6494) < 1e-3
    ref_o, ref_lse = oracle.combine(op.numpy(), mp.numpy(), lp.numpy())
    assert np.max(np.abs(host(o) - ref_o)) < 1e-6
    assert abs(float(lse.cpu()[0, 0, 0]) - ref_lse[0, 0, 0]) < 1e-5


def test_gpu_rejects_bad_arguments():
    fa = fa_mod()
    q = torch.zeros((1, 3, 4, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 2, 4, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FaError) as e:
        fa.attention(q, k, k)
    assert e.value.status == -1
    q = torch.zeros((1, 2, 4, 80), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 2, 4, 80), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FaError) as e:
        fa.attention(q, k, k)
    assert e.value.status == -2


# Soft-capped scores are bounded by the cap, so up to a cap of 60 the kernel
# keeps a fixed reference maximum of 0 (no running maximum, no rescale);
# above it the running maximum is used.  Both must give the exact result,
# also with the scores saturated near +-cap: Q and K are scaled by 3 (scores
# reach a few hundred before the cap), V keeps the workloads' N(0, 1) values
# the absolute O tolerance is set for.
@pytest.mark.parametrize("cap", [1.0, 50.0, 60.0, 61.0, 200.0])
@pytest.mark.parametrize("d", [64, 128])
def test_bf16_softcap_fixed_and_running_maximum(cap, d):
    print(f"case softcap cap={cap} d={d}", flush=True)
    inp = rand_inputs(2, 4, 2, 200, 333, d, seed=int(cap) + d, dtype="bf16")
    inp["q"], inp["k"] = (wl.round_bf16(inp[n] * np.float32(3.0)) for n in ("q", "k"))
    parity(inp, "bf16", 1.0, causal=True, softcap=cap, what=f"cap={cap}")
    parity(inp, "bf16", 1.0 / math.sqrt(d), causal=True, window=50, softcap=cap, what=f"cap={cap} window")
