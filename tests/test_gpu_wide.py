"""Parity of the 64-rows-per-wave bf16 kernel (d = 128, grids of at least
512 blocks of 256 query rows) with the fp64 oracle, on every row.

The shapes cover what the kernel's block pairing and masking distinguish:
K/V head counts that are and are not multiples of 8 (XCD-ordered or linear
block order), even and odd heads per K/V head (pairs inside a K/V group or
across K/V heads), an odd number of head slots (a workgroup whose second
group has no block), ragged query and key tails, cross attention with
Nq != Nk, rows that see no key, windows on alternate heads with a soft-cap
(the fixed-maximum path) and above the fixed-maximum threshold, a negative
scale, and scores large enough to move the running maximum often.
Tolerances as in test_gpu_parity.py (bf16: max |dO| <= 2e-2, mean <= 2e-3,
lse <= 1e-4 relative).
"""
import math

import numpy as np
import pytest

import oracle
from online_softmax_tiled_amd import workloads as wl

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN, BF16_LSE = 2e-2, 2e-3, 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import online_softmax_tiled_amd as fa
    fa.load_library()
    yield


def blocks(B, H, Nq):
    return B * H * ((Nq + 255) // 256)


def run_case(B, H, Hkv, Nq, Nk, seed, scale=None, causal=True, head_window=None, softcap=0.0, scale_in=1.0,
             v_scale=1.0):
    import online_softmax_tiled_amd as fa
    d = 128
    assert blocks(B, H, Nq) >= 512, "shape too small for the wide kernel"
    w = wl.Workload("wide", B, H, Hkv, Nq, Nk, d, "bf16", causal, 1.0, seed)
    inp = wl.generate(w)
    if scale_in != 1.0:
        # Q and K only: V keeps the N(0, 1) values the absolute O tolerance is set for.
        inp["q"], inp["k"] = (wl.round_bf16(inp[n] * np.float32(scale_in)) for n in ("q", "k"))
    if v_scale != 1.0:
        inp["v"] = wl.round_bf16(inp["v"] * np.float32(v_scale))
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    q, k, v = (torch.from_numpy(inp[n]).to(torch.bfloat16).cuda() for n in "qkv")
    o = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    fa.attention(q, k, v, scale=scale, causal=causal, head_window=head_window, softcap=softcap, out=o, lse=lse)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    ref = oracle.attention(inp["q"], inp["k"], inp["v"], scale, causal=causal, head_window=head_window,
                           softcap=softcap)
    assert np.all(np.isfinite(o)), "non-finite output"
    err = np.abs(o - ref["o"])
    assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN, f"|dO| max {err.max():.3g} mean {err.mean():.3g}"
    fin = np.isfinite(ref["lse"])
    assert np.array_equal(fin, np.isfinite(lse)), "-inf pattern of lse differs"
    assert np.all(o[~fin] == 0.0), "rows with no visible key must be 0"
    rel = np.abs(lse[fin] - ref["lse"][fin]) / np.maximum(1.0, np.abs(ref["lse"][fin]))
    assert rel.size == 0 or rel.max() <= BF16_LSE, f"lse rel err {rel.max():.3g}"
    return err


CASES = {
    # B, H, Hkv, Nq, Nk, extra
    "causal_mha_ragged": (4, 32, 32, 1100, 1100, {}),                      # XCD order, pairs across K/V heads
    "gqa_windows_softcap": (2, 32, 8, 2100, 2100,                          # pairs inside a K/V group
                            dict(head_window=[300 if h % 2 == 0 else 0 for h in range(32)], softcap=50.0)),
    # Scores up to a few hundred, capped at 70 (running maximum).  Rows are
    # then dominated by few keys whose weights, with the lazily moved
    # reference maximum, are not exactly 1, so their bf16 rounding (2^-9)
    # reaches O whole; V is scaled to |v| < 2 so that this rounding and O's
    # own stay inside the absolute tolerance.
    "gqa_softcap_running_max": (2, 32, 8, 2100, 2100, dict(softcap=70.0, scale_in=3.0, v_scale=0.3)),
    "xcd_odd_slots": (1, 24, 8, 6000, 6000, {}),                          # 3 head slots per XCD: one lone block
    "cross_noncausal": (8, 16, 16, 1050, 777, dict(causal=False)),
    "odd_slots_linear": (3, 45, 15, 1300, 1300, {}),                       # 135 head slots: one lone block
    "odd_rep_even_units": (2, 30, 10, 2300, 2300, dict(head_window=[200] * 30)),  # rep 3, 20 units
    "more_queries_than_keys": (2, 64, 16, 1200, 700, {}),                  # first 500 rows see nothing
    "negative_scale": (4, 32, 8, 1024, 1024, dict(scale=-0.05)),
    "large_scores": (4, 32, 32, 1000, 1000, dict(scale=40.0 / math.sqrt(128))),
}


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", list(CASES))
def test_wide_kernel_parity(name):
    B, H, Hkv, Nq, Nk, kw = CASES[name]
    print(f"case wide {name}: B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} {kw}", flush=True)
    kw = dict(kw)
    err = run_case(B, H, Hkv, Nq, Nk, seed=sum(map(ord, name)), **kw)
    print(f"  max |dO| {err.max():.3e} mean {err.mean():.3e}", flush=True)
