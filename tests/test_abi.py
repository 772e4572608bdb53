"""The C ABI library: it loads, exports what include/fa_mi355x.h declares,
its struct layout matches the binding, and argument validation rejects bad
calls before any HIP work (these calls never reach the GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

from online_softmax_tiled_amd import fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa_mi355x.h")

FAKE = 0x1000  # a non-null address that validation-failing calls never touch


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)))


def test_library_is_built_and_loads():
    assert os.path.exists(fa.library_path()), "run python -m online_softmax_tiled_amd.build"
    fa.load_library()


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(fa.EXPORTED), names
    lib = ctypes.CDLL(fa.library_path())
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", fa.library_path()], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", out, flags=re.M), n


def test_status_strings():
    assert fa.fa_status_string(0) == "FA_OK"
    for s in (-1, -2, -3):
        assert fa.fa_status_string(s).startswith("FA_ERR")
    assert "unknown" in fa.fa_status_string(7)


def test_struct_layout_matches_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "fa_mi355x.h"\n'
                   "int main(void){printf(\"%zu %zu %zu %zu\\n\", sizeof(fa_fwd_args),"
                   " offsetof(fa_fwd_args, scale), offsetof(fa_fwd_args, head_window),"
                   " offsetof(fa_fwd_args, stream));return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", f"-I{os.path.join(ROOT, 'include')}", str(src), "-o", str(exe)], check=True)
    vals = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()]
    A = fa.FwdArgs
    assert vals == [ctypes.sizeof(A), A.scale.offset, A.head_window.offset, A.stream.offset]


def call_fwd(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, H=4, Hkv=2, Nq=8, Nk=8, d=64,
             scale=0.125, causal=0, window=0, softcap=0.0, stream=FAKE)
    a.update(over)
    lib = fa.load_library()
    return lib.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Hkv"], a["Nq"], a["Nk"],
                      a["d"], a["scale"], a["causal"], a["window"], a["softcap"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(H=3), fa.FA_ERR_INVALID_ARG),                 # H % Hkv != 0
    (dict(Hkv=0), fa.FA_ERR_INVALID_ARG),
    (dict(B=-1), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=-5), fa.FA_ERR_INVALID_ARG),
    (dict(window=4), fa.FA_ERR_INVALID_ARG),            # window needs causal
    (dict(window=-1, causal=1), fa.FA_ERR_INVALID_ARG),
    (dict(softcap=-1.0), fa.FA_ERR_INVALID_ARG),
    (dict(softcap=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(k=None), fa.FA_ERR_INVALID_ARG),
    (dict(o=None), fa.FA_ERR_INVALID_ARG),
    (dict(d=48), fa.FA_ERR_UNSUPPORTED),
    (dict(d=256), fa.FA_ERR_UNSUPPORTED),
    # sizes whose products do not fit 64 bits are refused, not wrapped
    (dict(Nq=1 << 62), fa.FA_ERR_UNSUPPORTED),
    (dict(Nk=1 << 62), fa.FA_ERR_UNSUPPORTED),
    (dict(B=1 << 40, Nq=1 << 40, Nk=1 << 20), fa.FA_ERR_UNSUPPORTED),
    (dict(B=1 << 30, H=8, Hkv=2), fa.FA_ERR_UNSUPPORTED),
])
def test_fwd_validation(over, status):
    assert call_fwd(**over) == status


def test_empty_is_a_no_op_without_touching_pointers():
    # No query rows: nothing to do, so NULL tensors are fine and nothing runs.
    assert call_fwd(Nq=0, q=None, o=None) == fa.FA_OK
    assert call_fwd(B=0, q=None, k=None, v=None, o=None) == fa.FA_OK


def test_splitkv_and_combine_validation():
    lib = fa.load_library()
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4, 2, 1, 64, 64, 0.1, 0, 0, 0.0]
    assert lib.fa_fwd_splitkv(*base, 0, FAKE) == fa.FA_ERR_INVALID_ARG      # num_splits < 1
    b2 = list(base); b2[4] = None
    assert lib.fa_fwd_splitkv(*b2, 4, FAKE) == fa.FA_ERR_INVALID_ARG        # NULL m_part
    b3 = list(base); b3[11] = 80
    assert lib.fa_fwd_splitkv(*b3, 4, FAKE) == fa.FA_ERR_UNSUPPORTED        # d = 80
    c = [FAKE, FAKE, FAKE, FAKE, None, 1, 4, 1, 64]
    assert lib.fa_combine(*c, 0, fa.FA_DTYPE_BF16, FAKE) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_combine(*c, 4, 7, FAKE) == fa.FA_ERR_INVALID_ARG            # unknown dtype
    c2 = list(c); c2[3] = None
    assert lib.fa_combine(*c2, 4, fa.FA_DTYPE_BF16, FAKE) == fa.FA_ERR_INVALID_ARG
    c3 = list(c); c3[8] = 96
    assert lib.fa_combine(*c3, 4, fa.FA_DTYPE_FP32, FAKE) == fa.FA_ERR_UNSUPPORTED
    assert lib.fa_combine(None, None, None, None, None, 0, 4, 1, 64, 4, fa.FA_DTYPE_FP32, FAKE) == fa.FA_OK


def test_fwd_ex_validation():
    lib = fa.load_library()
    hw = (ctypes.c_int32 * 4)(0, 16, 0, 16)
    a = fa.FwdArgs(fa.FA_DTYPE_BF16, FAKE, FAKE, FAKE, FAKE, None, 1, 4, 2, 8, 8, 64, 0.1, 0, 0, 0.0,
                   ctypes.cast(hw, ctypes.POINTER(ctypes.c_int32)), FAKE)
    assert lib.fa_fwd_ex(ctypes.byref(a)) == fa.FA_ERR_INVALID_ARG          # per-head window, not causal
    hw2 = (ctypes.c_int32 * 4)(0, -3, 0, 16)
    a.causal = 1
    a.head_window = ctypes.cast(hw2, ctypes.POINTER(ctypes.c_int32))
    assert lib.fa_fwd_ex(ctypes.byref(a)) == fa.FA_ERR_INVALID_ARG          # negative entry
    a.dtype = 5
    assert lib.fa_fwd_ex(ctypes.byref(a)) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_fwd_ex(None) == fa.FA_ERR_INVALID_ARG
    big = (ctypes.c_int32 * 512)()
    a2 = fa.FwdArgs(fa.FA_DTYPE_BF16, FAKE, FAKE, FAKE, FAKE, None, 1, 512, 512, 8, 8, 64, 0.1, 1, 0, 0.0,
                    ctypes.cast(big, ctypes.POINTER(ctypes.c_int32)), FAKE)
    assert lib.fa_fwd_ex(ctypes.byref(a2)) == fa.FA_ERR_UNSUPPORTED         # H > FA_MAX_HEAD_WINDOWS


def test_rolling_cache_validation():
    # every rejected call returns before any launch, so it runs without a GPU
    lib = fa.load_library()
    app = [FAKE, FAKE, FAKE, FAKE, 2, 2, 3, 64]           # k_new, v_new, k_cache, v_cache, B, Hkv, T, d
    assert lib.fa_kv_append(*app, -1, 8, 4, FAKE) == fa.FA_ERR_INVALID_ARG      # pos < 0
    assert lib.fa_kv_append(*app, 5, 0, 4, FAKE) == fa.FA_ERR_INVALID_ARG       # window < 1
    assert lib.fa_kv_append(*app, 5, 8, -1, FAKE) == fa.FA_ERR_INVALID_ARG      # sinks < 0
    a2 = list(app); a2[2] = None
    assert lib.fa_kv_append(*a2, 5, 8, 4, FAKE) == fa.FA_ERR_INVALID_ARG        # NULL cache
    a3 = list(app); a3[7] = 80
    assert lib.fa_kv_append(*a3, 5, 8, 4, FAKE) == fa.FA_ERR_UNSUPPORTED        # d = 80
    a4 = list(app); a4[6] = 0; a4[0] = a4[1] = a4[2] = a4[3] = None
    assert lib.fa_kv_append(*a4, 5, 8, 4, FAKE) == fa.FA_OK                     # no tokens: no-op
    a5 = list(app); a5[4] = a5[5] = a5[6] = 1 << 30
    assert lib.fa_kv_append(*a5, 5, 8, 4, FAKE) == fa.FA_ERR_UNSUPPORTED        # B*Hkv*T beyond 2^63
    dec = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 64]  # q, caches, partials, B, H, Hkv, d
    assert lib.fa_decode_rolling(*dec, 10, 8, 4, 0.1, 0.0, 0, FAKE) == fa.FA_ERR_INVALID_ARG   # num_splits
    assert lib.fa_decode_rolling(*dec, -2, 8, 4, 0.1, 0.0, 4, FAKE) == fa.FA_ERR_INVALID_ARG   # pos
    assert lib.fa_decode_rolling(*dec, 10, 0, 4, 0.1, 0.0, 4, FAKE) == fa.FA_ERR_INVALID_ARG   # window
    d2 = list(dec); d2[7] = 3
    assert lib.fa_decode_rolling(*d2, 10, 8, 4, 0.1, 0.0, 4, FAKE) == fa.FA_ERR_INVALID_ARG    # H % Hkv
    d3 = list(dec); d3[4] = None
    assert lib.fa_decode_rolling(*d3, 10, 8, 4, 0.1, 0.0, 4, FAKE) == fa.FA_ERR_INVALID_ARG    # NULL m_part
    assert lib.fa_decode_rolling(*dec, 10, 8, 4, float("nan"), 0.0, 4, FAKE) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_decode_rolling(*dec, 10, 8, 4, 0.1, -2.0, 4, FAKE) == fa.FA_ERR_INVALID_ARG
    d4 = list(dec); d4[9] = 96
    assert lib.fa_decode_rolling(*d4, 10, 8, 4, 0.1, 0.0, 4, FAKE) == fa.FA_ERR_UNSUPPORTED


def test_softmax_validation():
    lib = fa.load_library()
    F, B = fa.FA_DTYPE_FP32, fa.FA_DTYPE_BF16
    assert lib.fa_softmax(FAKE, FAKE, None, -1, 8, F, FAKE) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_softmax(FAKE, FAKE, None, 4, -8, F, FAKE) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_softmax(FAKE, FAKE, None, 4, 8, 9, FAKE) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_softmax(None, FAKE, None, 4, 8, B, FAKE) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_softmax(FAKE, None, None, 4, 8, B, FAKE) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_softmax(None, None, None, 0, 8, F, FAKE) == fa.FA_OK          # no rows: no-op
    assert lib.fa_softmax(FAKE, FAKE, None, 1 << 31, 8, F, FAKE) == fa.FA_ERR_UNSUPPORTED
    t = [FAKE, FAKE, FAKE, None, 4, 100]
    assert lib.fa_softmax_topk(*t, 0, F, FAKE) == fa.FA_ERR_INVALID_ARG        # k < 1
    assert lib.fa_softmax_topk(*t, fa.FA_MAX_TOPK + 1, F, FAKE) == fa.FA_ERR_INVALID_ARG
    t2 = list(t); t2[5] = 5
    assert lib.fa_softmax_topk(*t2, 6, F, FAKE) == fa.FA_ERR_INVALID_ARG       # k > n
    t3 = list(t); t3[2] = None
    assert lib.fa_softmax_topk(*t3, 4, F, FAKE) == fa.FA_ERR_INVALID_ARG       # NULL indices
    assert lib.fa_softmax_topk(*t, 4, 7, FAKE) == fa.FA_ERR_INVALID_ARG        # unknown dtype
    t4 = list(t); t4[5] = 1 << 31
    assert lib.fa_softmax_topk(*t4, 4, B, FAKE) == fa.FA_ERR_UNSUPPORTED


def call_fp8(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, H=4, Hkv=2, Nq=8, Nk=8, d=128, scale=0.125,
             qd=1.0, kd=1.0, vd=1.0, causal=0, window=0, stream=FAKE)
    a.update(over)
    return fa.load_library().fa_fwd_fp8(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Hkv"],
                                        a["Nq"], a["Nk"], a["d"], a["scale"], a["qd"], a["kd"], a["vd"],
                                        a["causal"], a["window"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(qd=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(kd=-2.0), fa.FA_ERR_INVALID_ARG),
    (dict(vd=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(vd=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=3e38, qd=3e38), fa.FA_ERR_INVALID_ARG),   # score factor beyond fp32
    (dict(H=3), fa.FA_ERR_INVALID_ARG),
    (dict(window=4), fa.FA_ERR_INVALID_ARG),
    (dict(v=None), fa.FA_ERR_INVALID_ARG),
    (dict(d=32), fa.FA_ERR_UNSUPPORTED),                  # fp8 kernels: d in {64, 128}
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
])
def test_fp8_validation(over, status):
    assert call_fp8(**over) == status


def test_fp8_empty_is_a_no_op():
    assert call_fp8(Nq=0, q=None, o=None) == fa.FA_OK


def test_binding_rejects_mis_sized_output_buffers():
    # A caller-supplied output must match the shape and dtype the kernel
    # writes, be contiguous and live on the device; the binding checks this
    # before any launch (here on host tensors, which it also rejects).
    torch = pytest.importorskip("torch")
    good = fa._buffer(None, (2, 3), torch.float32, "cpu", "out")
    assert tuple(good.shape) == (2, 3) and good.dtype == torch.float32
    for bad in (torch.empty(2, 4), torch.empty(2, 3, dtype=torch.float64), torch.empty(3, 2).t(),
                torch.empty(2, 3)):
        with pytest.raises(ValueError, match="out must be"):
            fa._buffer(bad, (2, 3), torch.float32, "cpu", "out")


@pytest.mark.parametrize("which", ["q", "k", "v", "o"])
def test_misaligned_tensor_pointers_are_refused(which):
    # Every kernel moves 16 bytes per lane from the tensor base pointers: an
    # address off by one bf16 element is refused before any launch.
    assert call_fwd(**{which: FAKE + 2}) == fa.FA_ERR_INVALID_ARG
    assert call_fwd(**{which: FAKE + 8}) == fa.FA_ERR_INVALID_ARG
    assert call_fp8(**{which: FAKE + 4}) == fa.FA_ERR_INVALID_ARG


def test_misaligned_row_arrays_and_partials_are_refused():
    lib = fa.load_library()
    assert call_fwd(lse=FAKE + 2) == fa.FA_ERR_INVALID_ARG
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4, 2, 1, 64, 64, 0.1, 0, 0, 0.0]
    for i, off in ((3, 4), (4, 2), (5, 1)):              # o_part (16-byte), m_part, l_part (4-byte)
        b = list(base); b[i] = FAKE + off
        assert lib.fa_fwd_splitkv(*b, 4, FAKE) == fa.FA_ERR_INVALID_ARG
    c = [FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4, 1, 64]
    assert lib.fa_combine(*c[:3], FAKE + 1, *c[4:], 4, fa.FA_DTYPE_BF16, FAKE) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_combine(*c[:3], FAKE + 2, *c[4:], 4, fa.FA_DTYPE_FP32, FAKE) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_combine(FAKE + 2, *c[1:], 4, fa.FA_DTYPE_FP32, FAKE) == fa.FA_ERR_INVALID_ARG
    app = [FAKE, FAKE, FAKE + 8, FAKE, 2, 2, 3, 64]
    assert lib.fa_kv_append(*app, 5, 8, 4, FAKE) == fa.FA_ERR_INVALID_ARG


def test_binding_checks_head_window_length_and_alignment():
    # The library reads head_window[h] for all H heads: a shorter list is
    # refused by the binding before the call.
    with pytest.raises(ValueError, match="one per query head"):
        fa.fa_fwd_ex(fa.FA_DTYPE_BF16, FAKE, FAKE, FAKE, FAKE, None, 1, 4, 2, 8, 8, 64, 0.1, 1, 0, 0.0,
                     head_window=[0, 16, 0])
    torch = pytest.importorskip("torch")
    x = torch.empty(40, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="aligned"):
        fa._check_aligned(x[1:], 16, "q")
    fa._check_aligned(x[8:], 16, "q")


def test_static_scratch_entry_point_validation():
    # Refused before any HIP call: these run without a GPU.
    lib = fa.load_library()
    args = [FAKE, FAKE, FAKE, FAKE, None, 4, 32, 8, 32, 64, 128, 0.1, 0, 0, 0.0]
    assert lib.fa_splitkv_attention_static(*args, 0, fa.FA_DTYPE_BF16, FAKE) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_splitkv_attention_static(*args, 4, 9, FAKE) == fa.FA_ERR_INVALID_ARG   # out dtype
    # 4096 rows x 64 splits x (128 + 2) fp32 partials exceed the 8 MiB scratch
    assert lib.fa_splitkv_attention_static(*args, 64, fa.FA_DTYPE_BF16, FAKE) == fa.FA_ERR_SCRATCH_LIMIT
    assert "scratch" in fa.fa_status_string(fa.FA_ERR_SCRATCH_LIMIT)
    a2 = list(args); a2[2] = None
    assert lib.fa_splitkv_attention_static(*a2, 4, fa.FA_DTYPE_BF16, FAKE) == fa.FA_ERR_INVALID_ARG
