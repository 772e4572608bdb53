"""Parity of the small-grid bf16 kernel (4 waves per 32 query rows, keys
split among them, merged in LDS) with the fp64 oracle, on every row.

It takes unsplit bf16 launches whose 128-row workgroups would number under
256 and that have at least 256 keys.  The shapes cover what its key split
and merge distinguish: d = 32, 64 and 128; key counts that are and are not
multiples of the 32-key step and of four steps; ragged query tiles; causal
blocks whose four waves get unequal or empty key ranges; windows on
alternate heads (a wave may see no key of its quarter); a soft-cap; GQA;
rows that see no key at all; a negative scale; and scores large enough to
move the running maximum often.  Tolerances as in test_gpu_parity.py.
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


def takes_splitk(B, H, Nq, Nk):
    return B * H * ((Nq + 127) // 128) < 256 and Nk >= 256


CASES = {
    # B, H, Hkv, Nq, Nk, d, extra
    "c2_shape_d64": (1, 8, 8, 1024, 1024, 64, dict(causal=False)),
    "d32_ragged": (1, 4, 2, 77, 1000, 32, dict(causal=False)),
    "d128_causal_ragged": (2, 4, 4, 333, 333, 128, dict(causal=True)),
    "d64_causal_gqa": (1, 8, 2, 700, 700, 64, dict(causal=True)),
    "d128_windows_softcap": (1, 4, 2, 600, 600, 128,
                             dict(causal=True, head_window=[100, 0, 100, 0], softcap=30.0)),
    "d64_more_queries_than_keys": (1, 4, 4, 500, 300, 64, dict(causal=True)),
    "d64_negative_scale": (1, 6, 3, 256, 513, 64, dict(causal=False, scale=-0.06)),
    "d128_large_scores": (1, 4, 4, 200, 1500, 128, dict(causal=False, scale=40.0 / math.sqrt(128))),
    "d32_keys_not_step_multiple": (2, 2, 1, 64, 257, 32, dict(causal=False)),
}


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", list(CASES))
def test_splitk_kernel_parity(name):
    import online_softmax_tiled_amd as fa
    B, H, Hkv, Nq, Nk, d, kw = CASES[name]
    kw = dict(kw)
    assert takes_splitk(B, H, Nq, Nk), "shape would not take the small-grid kernel"
    print(f"case splitk {name}: B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} {kw}", flush=True)
    causal = kw.pop("causal")
    scale = kw.pop("scale", 1.0 / math.sqrt(d))
    head_window = kw.pop("head_window", None)
    softcap = kw.pop("softcap", 0.0)
    w = wl.Workload("splitk", B, H, Hkv, Nq, Nk, d, "bf16", causal, scale, sum(map(ord, name)))
    inp = wl.generate(w)
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
    print(f"  max |dO| {err.max():.3e} mean {err.mean():.3e}", flush=True)
    assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN, f"|dO| max {err.max():.3g} mean {err.mean():.3g}"
    fin = np.isfinite(ref["lse"])
    assert np.array_equal(fin, np.isfinite(lse)), "-inf pattern of lse differs"
    assert np.all(o[~fin] == 0.0), "rows with no visible key must be 0"
    rel = np.abs(lse[fin] - ref["lse"][fin]) / np.maximum(1.0, np.abs(ref["lse"][fin]))
    assert rel.size == 0 or rel.max() <= BF16_LSE, f"lse rel err {rel.max():.3g}"
