"""How the fp8 matrix instruction accumulates, pinned on the GPU.

The fp8 attention tolerances (test_gpu_fp8.py) rest on a model of
v_mfma_f32_32x32x64_f8f6f4 with E4M3 operands: products of two E4M3 values
are exact; they are added in groups of 8 consecutive k in a fixed-point
window about 13 bits below the group's largest product (a product 2^13 below
it still counts, one 2^14 below is dropped); the group sums are then added
in fp32.  So a 64-term dot product is exact when the products lie within
2^6 of one another, and otherwise off by at most 7 * 2^-13 (< EPS_MM =
2^-10) of the sum of |products|.

These tests measure that model with tests/probes/libfp8_mfma_probe.so (one
MFMA per case whose result element is sum_k a_k b_k) against exact sums of
the decoded products (oracle/fp8.py decodes E4M3; the sums are fp64, exact
for these magnitudes).  They print what they measure; the figures are kept
in profiles/fp8_mfma_accumulation.md.
"""
import ctypes
import math
import os

import numpy as np
import pytest

from oracle import fp8 as ofp8

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes", "libfp8_mfma_probe.so")
ONE, TWO_M6, TWO_M7, TWO_M8 = 0x38, 0x08, 0x04, 0x02  # E4M3 codes of 1, 2^-6, 2^-7, 2^-8
EPS_MM = 2.0 ** -10


@pytest.fixture(scope="module")
def probe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(LIB), f"{LIB} missing: run __graft_entry__.build() (tests/probes/build.py)"
    lib = ctypes.CDLL(LIB)
    lib.fp8_mfma_probe.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.fp8_mfma_probe.restype = ctypes.c_int

    def run(a_codes, b_codes):
        a = torch.from_numpy(np.ascontiguousarray(a_codes, dtype=np.uint8)).cuda()
        b = torch.from_numpy(np.ascontiguousarray(b_codes, dtype=np.uint8)).cuda()
        n = a.shape[0]
        out = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
        assert lib.fp8_mfma_probe(a.data_ptr(), b.data_ptr(), out.data_ptr(), n, None) == 0
        torch.cuda.synchronize()
        return out.cpu().numpy().astype(np.float64)
    return run


def exact(a_codes, b_codes):
    return (ofp8.e4m3_value(a_codes) * ofp8.e4m3_value(b_codes)).sum(axis=1)


def case(pairs):
    """One case from {k: (a_code, b_code)}; other k hold zero products."""
    a = np.zeros(64, dtype=np.uint8)
    b = np.zeros(64, dtype=np.uint8)
    for k, (ca, cb) in pairs.items():
        a[k], b[k] = ca, cb
    return a, b


def test_window_inside_a_group(probe):
    """1 + 2^-13 in one group keeps the small product; 1 + 2^-14 drops it."""
    rows = [case({0: (ONE, ONE), 1: (TWO_M7, TWO_M6)}),   # 1 + 2^-13
            case({0: (ONE, ONE), 1: (TWO_M8, TWO_M6)}),   # 1 + 2^-14
            case({0: (ONE, ONE), 7: (TWO_M8, TWO_M6)})]   # same group, last slot
    a = np.stack([r[0] for r in rows])
    b = np.stack([r[1] for r in rows])
    got = probe(a, b)
    print(f"1 + 2^-13 -> {got[0]!r}; 1 + 2^-14 (k = 1) -> {got[1]!r}; 1 + 2^-14 (k = 7) -> {got[2]!r}", flush=True)
    assert got[0] == 1.0 + 2.0 ** -13
    assert got[1] == 1.0
    assert got[2] == 1.0


def test_groups_are_eight_consecutive_k(probe):
    """A product 2^-14 below the largest survives when it is in another group of 8."""
    rows = [case({0: (ONE, ONE), 8: (TWO_M8, TWO_M6)}),
            case({7: (ONE, ONE), 8: (TWO_M8, TWO_M6)}),
            case({31: (ONE, ONE), 32: (TWO_M8, TWO_M6)}),
            case({0: (ONE, ONE), 63: (TWO_M8, TWO_M6)})]
    a = np.stack([r[0] for r in rows])
    b = np.stack([r[1] for r in rows])
    got = probe(a, b)
    print("different groups, 1 + 2^-14 ->", [repr(g) for g in got], flush=True)
    assert np.all(got == 1.0 + 2.0 ** -14)


def test_exact_within_two_to_the_six(probe):
    """All 64 products within [1, 64): the sum is exact."""
    rng = np.random.default_rng(71)
    # E4M3 normals in [1, 8): exponent field 7..9 (codes 0x38..0x4f), random signs.
    n = 2000
    a = rng.integers(0x38, 0x50, size=(n, 64), dtype=np.uint8) | (rng.integers(0, 2, size=(n, 64)) << 7).astype(np.uint8)
    b = rng.integers(0x38, 0x50, size=(n, 64), dtype=np.uint8) | (rng.integers(0, 2, size=(n, 64)) << 7).astype(np.uint8)
    got = probe(a, b)
    ref = exact(a, b)
    bad = int(np.count_nonzero(got != ref))
    print(f"{n} cases, products within [1, 64): {bad} differ from the exact sum", flush=True)
    assert bad == 0


def test_full_range_error_bound(probe):
    """Random E4M3 codes over the whole range: error <= 7 * 2^-13 of sum |products|."""
    rng = np.random.default_rng(72)
    n = 4000
    codes = np.array([c for c in range(256) if c not in (0x7f, 0xff)], dtype=np.uint8)
    a = rng.choice(codes, size=(n, 64))
    b = rng.choice(codes, size=(n, 64))
    got = probe(a, b)
    pa, pb = ofp8.e4m3_value(a), ofp8.e4m3_value(b)
    ref = (pa * pb).sum(axis=1)
    mag = np.abs(pa * pb).sum(axis=1)
    ratio = np.abs(got - ref) / np.where(mag > 0, mag, 1.0)
    worst = float(ratio.max())
    print(f"{n} full-range cases: max |error| / sum|products| = {worst:.3e} "
          f"(2^{math.log2(worst) if worst > 0 else float('-inf'):.2f}); bound 7*2^-13 = {7 * 2.0 ** -13:.3e}; "
          f"exact in {int(np.count_nonzero(ratio == 0))} of {n}", flush=True)
    assert worst <= 7 * 2.0 ** -13
    assert worst < EPS_MM
