"""Pins of the fp8 oracle (oracle/fp8.py): the E4M3 decoder against the
format's defining values and torch's own float8_e4m3fn conversion, and
attention of fp8 inputs against closed forms.  CPU only."""
import math

import numpy as np
import pytest

from oracle import fp8 as ofp8
from online_softmax_tiled_amd import workloads as wl

torch = pytest.importorskip("torch")


def test_decoder_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = ofp8.e4m3_value(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x38, 1.0), (0xB8, -1.0), (0x40, 2.0), (0x30, 0.5), (0x7E, 448.0), (0xFE, -448.0),
    (0x08, 2.0 ** -6),          # smallest normal
    (0x07, 7 * 2.0 ** -9),      # largest subnormal
    (0x01, 2.0 ** -9),          # smallest subnormal
    (0x3F, 1.875), (0x39, 1.125), (0x77, 240.0),
])
def test_defining_values(code, value):
    assert ofp8.e4m3_value(np.array([code]))[0] == value


def test_nan_codes_and_negative_zero():
    v = ofp8.e4m3_value(np.array([0x7F, 0xFF, 0x80]))
    assert np.isnan(v[0]) and np.isnan(v[1])
    assert v[2] == 0.0 and np.signbit(v[2])
    assert np.sum(np.isnan(ofp8.e4m3_value(np.arange(256)))) == 2
    with pytest.raises(ValueError):
        ofp8.e4m3_value(np.array([256]))


def test_two_key_closed_form():
    # q = 1, keys 2 and 0 (times descales 0.5 and 2: their product is 1),
    # values 4 and 0.5 times 0.25: weights are the logistic of the score gap.
    d = 1
    q = np.full((1, 1, 1, d), 0x38, dtype=np.uint8)
    k = np.array([0x40, 0x00], dtype=np.uint8).reshape(1, 1, 2, d)
    v = np.array([0x48, 0x30], dtype=np.uint8).reshape(1, 1, 2, d)
    r = ofp8.attention_fp8(q, k, v, 0.5, 2.0, 0.25, 1.0)
    w0 = 1.0 / (1.0 + math.exp(-2.0))
    assert abs(r["o"][0, 0, 0, 0] - (w0 * 1.0 + (1 - w0) * 0.125)) < 1e-15
    assert abs(r["lse"][0, 0, 0] - (2.0 + math.log1p(math.exp(-2.0)))) < 1e-14


def test_descales_enter_as_products_and_linearly():
    w = wl.FP8_PREFILL.with_(B=1, H=2, Hkv=1, Nq=40, Nk=50, d=16)
    x = wl.generate_fp8(w)
    args = (x["q"], x["k"], x["v"])
    a = ofp8.attention_fp8(*args, 0.5, 0.25, 1.0, 0.3, causal=True)
    b = ofp8.attention_fp8(*args, 0.125, 1.0, 1.0, 0.3, causal=True)   # same product q_descale*k_descale
    c = ofp8.attention_fp8(*args, 1.0, 1.0, 1.0, 0.3 * 0.125, causal=True)  # folded into scale
    d = ofp8.attention_fp8(*args, 0.5, 0.25, 4.0, 0.3, causal=True)   # v_descale scales O
    assert np.allclose(a["o"], b["o"], rtol=1e-12, atol=0) and np.allclose(a["lse"], b["lse"], rtol=1e-12)
    assert np.allclose(a["o"], c["o"], rtol=1e-12, atol=0)
    assert np.allclose(4.0 * a["o"], d["o"], rtol=1e-12, atol=0)


def test_quantiser_round_trip_and_scale():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(10000).astype(np.float32) * 3
    codes, ds = wl.to_e4m3(x)
    back = ofp8.dequantise(codes, ds)
    # largest magnitude maps to 448; every value within half an E4M3 step
    # (relative 2^-4 in the normal range, 2^-10 * descale below it)
    assert np.max(np.abs(back)) == pytest.approx(np.max(np.abs(x)), rel=2 ** -4)
    err = np.abs(back - x)
    assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * ds) * (1 + 1e-6))
