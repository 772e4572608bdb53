"""Row softmax with the online normaliser (fa_softmax) and the fused softmax
top-k (fa_softmax_topk) against the fp64 oracle (oracle/softmax.py).

Tolerances: fp32 output |dy| <= 1e-5 * y (relative; every y is a single
exp times 1/d); bf16 output |dy| <= 2^-8 * y + 1e-30 plus the same fp32 part
(the result is rounded to bf16); lse |dlse| <= 1e-5 * max(1, |lse|).  Top-k
indices must equal the oracle's exactly (ties: lower index first); their
probabilities use the fp32 tolerance.
"""
import numpy as np
import pytest

from oracle import softmax as osm
from online_softmax_tiled_amd import workloads as wl

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


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


def logits(rows, n, seed, dtype, scale=3.0, shift=0.0):
    x = (np.random.default_rng(seed).standard_normal((rows, n)) * scale + shift).astype(np.float32)
    return wl.round_bf16(x) if dtype == "bf16" else x


def dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return (t.to(torch.bfloat16) if dtype == "bf16" else t).cuda()


def check_softmax(x, dtype, what):
    y_ref, lse_ref = osm.softmax(x)
    y, lse = fa_mod().softmax(dev(x, dtype), return_lse=True)
    torch.cuda.synchronize()
    y = y.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    tol = 1e-5 * y_ref + (2.0 ** -8 * y_ref + 1e-30 if dtype == "bf16" else 1e-37)
    bad = np.abs(y - y_ref) > tol
    assert not bad.any(), f"{what}: {bad.sum()} values off, worst rel {np.max(np.abs(y - y_ref) / (y_ref + 1e-300)):.3g}"
    assert np.all(np.abs(lse - lse_ref) <= 1e-5 * np.maximum(1.0, np.abs(lse_ref))), f"{what}: lse"


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("rows,n", [(3, 1), (7, 5), (5, 1000), (4, 4096), (6, 1001), (2, 33333), (3, 131072)])
def test_softmax_matches_oracle(dtype, rows, n):
    print(f"case softmax {dtype} rows={rows} n={n}", flush=True)
    check_softmax(logits(rows, n, seed=rows * 7 + n, dtype=dtype), dtype, f"{dtype} {rows}x{n}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_softmax_shifted_large_and_constant_rows(dtype):
    print(f"case softmax special rows {dtype}", flush=True)
    x = np.concatenate([logits(2, 2048, 1, dtype, scale=30.0, shift=500.0),   # large, shifted
                        logits(2, 2048, 2, dtype, scale=1e-3),                 # nearly uniform
                        np.full((1, 2048), -7.5, dtype=np.float32)])           # constant
    check_softmax(x, dtype, f"{dtype} special")


def check_topk(x, dtype, k, what):
    p_ref, i_ref, lse_ref = osm.softmax_topk(x, k)
    probs, idx, lse = fa_mod().softmax_topk(dev(x, dtype), k, return_lse=True)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    probs = probs.cpu().numpy().astype(np.float64)
    assert np.array_equal(idx, i_ref), f"{what}: indices differ in {np.sum(np.any(idx != i_ref, axis=1))} rows"
    assert np.all(np.abs(probs - p_ref) <= 1e-5 * p_ref + 1e-37), f"{what}: probabilities"
    assert np.all(np.abs(lse.cpu().numpy() - lse_ref) <= 1e-5 * np.maximum(1.0, np.abs(lse_ref)))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("k", [1, 5, 8, 64])
@pytest.mark.parametrize("rows,n", [(4, 64), (5, 999), (3, 8192), (2, 100003)])
def test_softmax_topk_matches_oracle(dtype, k, rows, n):
    print(f"case topk {dtype} k={k} rows={rows} n={n}", flush=True)
    check_topk(logits(rows, n, seed=k * 100 + n, dtype=dtype), dtype, k, f"{dtype} k={k} {rows}x{n}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_softmax_topk_ties_lower_index_first(dtype):
    # values on a coarse grid: many exact ties across lanes and waves
    print(f"case topk ties {dtype}", flush=True)
    x = np.round(logits(6, 20000, 5, "fp32") * 2.0) / 2.0
    check_topk(x.astype(np.float32), dtype, 64, f"{dtype} ties")
    z = np.zeros((2, 3000), dtype=np.float32)  # every value equal: columns 0..k-1
    check_topk(z, dtype, 16, f"{dtype} all equal")


def test_bench_shape_sampled():
    # the benchmark's configuration: 512 rows of 256000 fp32 logits; the
    # oracle checks a few rows of the same launch
    rows, n, k = 512, 256000, 8
    print("case softmax bench shape", flush=True)
    x = logits(rows, n, seed=9, dtype="fp32")
    xd = dev(x, "fp32")
    y, lse = fa_mod().softmax(xd, return_lse=True)
    probs, idx = fa_mod().softmax_topk(xd, k)
    torch.cuda.synchronize()
    pick = np.array([0, 1, 255, 256, 511])
    y_ref, lse_ref = osm.softmax(x[pick])
    yy = y.cpu().numpy()[pick].astype(np.float64)
    assert np.all(np.abs(yy - y_ref) <= 1e-5 * y_ref + 1e-37)
    assert np.allclose(lse.cpu().numpy()[pick], lse_ref, rtol=1e-5, atol=1e-5)
    p_ref, i_ref, _ = osm.softmax_topk(x[pick], k)
    assert np.array_equal(idx.cpu().numpy()[pick], i_ref)
    assert np.all(np.abs(probs.cpu().numpy()[pick] - p_ref) <= 1e-5 * p_ref)
