"""fa_splitkv_attention_static (split-KV attention whose partials live in
the library's fixed per-GPU scratch array; it allocates nothing) against
the entry points that take the partials as caller-allocated buffers,
fa_fwd_splitkv + fa_combine, through the C ABI: the same kernels on the
same inputs, so the outputs must agree bit for bit.  Two calls in a row,
the second with a smaller input (the scratch keeps the first call's
partials; every partial the second call reads is written by it first),
and a request beyond the scratch size refused without a launch."""
import ctypes
import math

import numpy as np
import pytest

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


def run_both(B, H, Hkv, Nq, Nk, d, S, seed, causal=False, window=0, softcap=0.0):
    import online_softmax_tiled_amd as fa
    from online_softmax_tiled_amd import fa as raw
    w = wl.Workload("static", B, H, Hkv, Nq, Nk, d, "bf16", causal, 1.0 / math.sqrt(d), seed)
    inp = wl.generate(w)
    q, k, v = (torch.from_numpy(inp[n]).to(torch.bfloat16).cuda() for n in "qkv")
    scale = 1.0 / math.sqrt(d)
    o1 = torch.full((B, H, Nq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    l1 = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device="cuda")
    lib = fa.load_library()
    rc = lib.fa_splitkv_attention_static(q.data_ptr(), k.data_ptr(), v.data_ptr(), o1.data_ptr(), l1.data_ptr(),
                                         B, H, Hkv, Nq, Nk, d, scale, int(causal), window, softcap, S,
                                         raw.FA_DTYPE_BF16, torch.cuda.current_stream().cuda_stream or None)
    assert rc == 0, fa.fa_status_string(rc)
    o2, l2 = fa.splitkv_attention(q, k, v, S, scale=scale, causal=causal, window=window, softcap=softcap)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2), "outputs differ from fa_fwd_splitkv + fa_combine"
    assert torch.equal(l1, l2), "lse differs from fa_fwd_splitkv + fa_combine"
    return o1


def test_static_scratch_matches_workspace_entry_points():
    print("case static scratch: decode shape, then a smaller mixed shape", flush=True)
    # 256 rows x 16 splits of d = 128: 2.1 MB of partials; MFMA split path for the second
    run_both(8, 32, 8, 1, 8192, 128, 16, seed=41)
    run_both(2, 8, 2, 40, 900, 64, 5, seed=42, causal=True, window=300, softcap=30.0)


def test_static_scratch_limit_is_refused():
    import online_softmax_tiled_amd as fa
    from online_softmax_tiled_amd import fa as raw
    lib = fa.load_library()
    # 4096 rows x 64 splits x 130 floats = 136 MB of partials > 8 MiB: refused before any launch
    q = torch.zeros((4, 32, 32, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((4, 8, 64, 128), dtype=torch.bfloat16, device="cuda")
    o = torch.zeros_like(q)
    rc = lib.fa_splitkv_attention_static(q.data_ptr(), k.data_ptr(), k.data_ptr(), o.data_ptr(), None, 4, 32, 8, 32,
                                         64, 128, 0.1, 0, 0, 0.0, 64, raw.FA_DTYPE_BF16, None)
    assert rc == raw.FA_ERR_SCRATCH_LIMIT
    assert "scratch" in fa.fa_status_string(rc)
    torch.cuda.synchronize()
    assert torch.count_nonzero(o) == 0
