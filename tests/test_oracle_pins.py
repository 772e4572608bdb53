"""Pins of the fp64 CPU oracle against what the pages and mathematics fix.

Nothing here compares the oracle with itself: every check is a value
printed on the pages, a closed form, an invariant of the definition, or an
independent brute force (Python ``decimal`` at 50 digits, a probability
formulation without any maximum subtraction, exp/ln from ``decimal``).
"""
import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle
from online_softmax_tiled_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- brute force
getcontext().prec = 50


def _dtanh(x: Decimal) -> Decimal:
    e = (2 * x).exp()
    return (e - 1) / (e + 1)


def _visible_keys(i, Nq, Nk, causal, W, sinks=0):
    """The keys a query sees, built as explicit position sets: every key, or
    the keys at or before the query's absolute position i + Nk - Nq, and of
    those only the W most recent when a window is set, together with the
    first ``sinks`` positions (attention sinks, Transformers & Math 16.6)."""
    p = i + Nk - Nq
    keys = set(range(Nk))
    if causal:
        keys &= set(range(0, p + 1))
    if W > 0:
        keys &= set(range(p - W + 1, p + 1)) | set(range(0, sinks))
    return sorted(keys)


def brute_force(q, k, v, scale, causal=False, head_window=None, softcap=0.0, sinks=0):
    """O and lse by the probability form p_j = 1 / sum_k exp(s_k - s_j),
    in 50-digit decimal arithmetic; no running or global maximum."""
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    hw = head_window if head_window is not None else [0] * H
    o = np.zeros((B, H, Nq, d))
    lse = np.full((B, H, Nq), -np.inf)
    sc = Decimal(float(scale))
    for b in range(B):
        for h in range(H):
            g = h // (H // Hkv)
            for i in range(Nq):
                keys = _visible_keys(i, Nq, Nk, causal, hw[h], sinks)
                if not keys:
                    continue
                s = {}
                for j in keys:
                    dot = sum(Decimal(float(q[b, h, i, c])) * Decimal(float(k[b, g, j, c]))
                              for c in range(d))
                    z = sc * dot
                    if softcap > 0:
                        kap = Decimal(float(softcap))
                        z = kap * _dtanh(z / kap)
                    s[j] = z
                for c in range(d):
                    acc = Decimal(0)
                    for j in keys:
                        pj = 1 / sum((s[t] - s[j]).exp() for t in keys)
                        acc += pj * Decimal(float(v[b, g, j, c]))
                    o[b, h, i, c] = float(acc)
                j0 = keys[0]
                lse[b, h, i] = float(s[j0] + sum((s[t] - s[j0]).exp() for t in keys).ln())
    return o, lse


def _rand(shape, rng, scale=1.0):
    return rng.standard_normal(shape) * scale


# ------------------------------------------------------------ worked example
def test_worked_example_direct():
    g = golden("worked_example.json")
    we = wl.worked_example(d=3)
    r = oracle.attention(we["q"], we["k"], we["v"], we["scale"])
    assert np.all(np.abs(r["o"] - g["expected_output"]) < g["tolerance"])
    # The weights are proportional to e^(ln i) = i, so the normaliser is
    # e^1000 * (1 + 2 + 3 + 4) and lse = 1000 + ln 10.
    assert abs(r["lse"][0, 0, 0] - (1000.0 + math.log(10.0))) < 1e-10


@pytest.mark.parametrize("tile", [1, 2, 4])
def test_worked_example_streaming_tiles(tile):
    g = golden("worked_example.json")
    assert tile in g["tile_sizes"]
    we = wl.worked_example(d=2)
    dense = oracle.attention(we["q"], we["k"], we["v"], we["scale"])["o"]
    r = oracle.attention(we["q"], we["k"], we["v"], we["scale"], tile=tile)
    assert np.all(np.abs(r["o"] - dense) < g["tolerance"])
    assert np.all(np.abs(r["o"] - g["expected_output"]) < g["tolerance"])


def test_worked_example_fp32_scores():
    # With fp32 inputs the scores are the fp32 roundings of 1000 + ln i; the
    # exact softmax of those rounded scores is the oracle's answer, checked
    # here in closed form: weights e^(s_i - s_1), values 10 i.
    we = wl.worked_example(d=2, dtype=np.float32)
    s = we["k"][0, 0, :, 0].astype(np.float64)
    w = [Decimal(float(x - s[0])).exp() for x in s]
    expect = float(sum(wi * Decimal(10 * (n + 1)) for n, wi in enumerate(w)) / sum(w))
    r = oracle.attention(we["q"], we["k"], we["v"], 1.0)
    assert abs(r["o"][0, 0, 0, 0] - expect) < 1e-11
    assert abs(expect - 29.99993039) < 1e-7


# ------------------------------------------------------------- closed forms
def test_single_key_returns_its_value():
    rng = np.random.default_rng(10)
    q, k, v = _rand((2, 3, 4, 5), rng), _rand((2, 3, 1, 5), rng), _rand((2, 3, 1, 5), rng)
    r = oracle.attention(q, k, v, 0.7)
    assert np.array_equal(r["o"], np.broadcast_to(v, r["o"].shape))
    s0 = 0.7 * np.einsum("bhid,bhd->bhi", q, k[:, :, 0, :])
    assert np.allclose(r["lse"], s0, rtol=0, atol=1e-12)


def test_causal_first_row_sees_only_first_key():
    rng = np.random.default_rng(11)
    q, k, v = (_rand((1, 2, 6, 4), rng) for _ in range(3))
    r = oracle.attention(q, k, v, 0.5, causal=True)
    assert np.array_equal(r["o"][:, :, 0, :], v[:, :, 0, :])


@pytest.mark.parametrize("Nq,Nk,causal,W", [
    (7, 7, False, 0), (7, 7, True, 0), (9, 9, True, 3), (3, 8, True, 0),
    (3, 8, True, 2), (8, 8, True, 1), (5, 11, False, 0)])
def test_uniform_scores_give_mean_of_visible_values(Nq, Nk, causal, W):
    # q = 0 makes every score 0, so each visible key weighs the same:
    # O = mean of the visible values, lse = ln(number visible).
    rng = np.random.default_rng(12)
    H = 2
    q = np.zeros((1, H, Nq, 3))
    k, v = _rand((1, H, Nk, 3), rng), _rand((1, H, Nk, 3), rng)
    r = oracle.attention(q, k, v, 1.3, causal=causal, window=W)
    for i in range(Nq):
        p = i + Nk - Nq
        hi = p + 1 if causal else Nk
        lo = max(0, p - W + 1) if W > 0 else 0
        n = hi - lo
        assert np.allclose(r["o"][0, :, i], v[0, :, lo:hi].mean(axis=1), atol=1e-14)
        assert abs(r["lse"][0, 0, i] - math.log(n)) < 1e-14


def test_softcap_matches_printed_values():
    g = golden("softcap_values.json")
    kap = g["kappa"]
    for case in g["cases"]:
        # One key with raw score z: lse is the capped score itself.
        q = np.zeros((1, 1, 1, 2)); q[..., 0] = case["logit"]
        k = np.zeros((1, 1, 1, 2)); k[..., 0] = 1.0
        v = np.ones((1, 1, 1, 2))
        r = oracle.attention(q, k, v, 1.0, softcap=kap)
        assert abs(r["lse"][0, 0, 0] - case["capped"]) <= case["tolerance"], case
    # 100 and 300 both land within a hair of the cap.
    for z in (100.0, 300.0):
        q = np.zeros((1, 1, 1, 1)); q[..., 0] = z
        r = oracle.attention(q, np.ones((1, 1, 1, 1)), np.ones((1, 1, 1, 1)), 1.0, softcap=kap)
        assert kap - 0.1 < r["lse"][0, 0, 0] < kap


def test_softcap_two_key_closed_form():
    kap = Decimal(50)
    z = [Decimal(60), Decimal(-20)]
    s = [kap * _dtanh(zi / kap) for zi in z]
    v1, v2 = Decimal(3), Decimal(-2)
    e1, e2 = s[0].exp(), s[1].exp()
    expect = float((e1 * v1 + e2 * v2) / (e1 + e2))
    q = np.array([[[[1.0]]]])
    k = np.array([[[[60.0], [-20.0]]]])
    v = np.array([[[[3.0], [-2.0]]]])
    r = oracle.attention(q, k, v, 1.0, softcap=50.0)
    assert abs(r["o"][0, 0, 0, 0] - expect) < 1e-13
    assert abs(r["lse"][0, 0, 0] - float((e1 + e2).ln())) < 1e-12


def test_empty_inputs():
    rng = np.random.default_rng(13)
    q, k, v = _rand((1, 2, 0, 4), rng), _rand((1, 2, 5, 4), rng), _rand((1, 2, 5, 4), rng)
    assert oracle.attention(q, k, v, 1.0)["o"].shape == (1, 2, 0, 4)
    q = _rand((1, 2, 3, 4), rng)
    k0, v0 = np.zeros((1, 2, 0, 4)), np.zeros((1, 2, 0, 4))
    r = oracle.attention(q, k0, v0, 1.0)
    assert np.all(r["o"] == 0) and np.all(np.isneginf(r["lse"]))
    assert np.all(r["l"] == 0) and np.all(np.isneginf(r["m"]))
    # Query rows that see no key at all: more queries than keys under a
    # causal mask leaves the first Nq - Nk rows with nothing visible.
    k, v = _rand((1, 2, 2, 4), rng), _rand((1, 2, 2, 4), rng)
    r = oracle.attention(_rand((1, 2, 4, 4), rng), k, v, 1.0, causal=True)
    assert np.all(r["o"][:, :, :2] == 0) and np.all(np.isneginf(r["lse"][:, :, :2]))


def test_rejects_invalid_arguments():
    rng = np.random.default_rng(14)
    q, k, v = _rand((1, 3, 2, 2), rng), _rand((1, 2, 2, 2), rng), _rand((1, 2, 2, 2), rng)
    with pytest.raises(ValueError):
        oracle.attention(q, k, v, 1.0)          # 3 query heads over 2 KV heads
    q = _rand((1, 2, 2, 2), rng)
    with pytest.raises(ValueError):
        oracle.attention(q, k, v, 1.0, window=2)  # window without causal


# ------------------------------------------------------------- brute force
BRUTE_CASES = [
    # B, H, Hkv, Nq, Nk, d, scale, causal, head_window, softcap
    (1, 1, 1, 4, 4, 3, 0.9, False, None, 0.0),
    (2, 2, 1, 3, 5, 2, 1.1, False, None, 0.0),
    (1, 4, 2, 5, 5, 3, 0.8, True, None, 0.0),
    (1, 2, 2, 6, 6, 2, 1.0, True, [2, 0], 0.0),
    (1, 4, 1, 3, 7, 2, 1.5, True, [3, 0, 1, 2], 0.0),
    (1, 2, 1, 4, 6, 3, 2.0, True, [0, 2], 1.5),
    (2, 2, 2, 2, 3, 4, 3.0, False, None, 2.0),
    (1, 1, 1, 5, 3, 2, 1.0, True, None, 0.0),
]


@pytest.mark.parametrize("n", range(len(BRUTE_CASES)))
def test_matches_decimal_brute_force(n):
    B, H, Hkv, Nq, Nk, d, scale, causal, hw, cap = BRUTE_CASES[n]
    rng = np.random.default_rng(100 + n)
    q, k, v = _rand((B, H, Nq, d), rng), _rand((B, Hkv, Nk, d), rng), _rand((B, Hkv, Nk, d), rng)
    o_ref, lse_ref = brute_force(q, k, v, scale, causal, hw, cap)
    r = oracle.attention(q, k, v, scale, causal=causal, head_window=hw, softcap=cap)
    assert np.allclose(r["o"], o_ref, rtol=0, atol=1e-13)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(r["lse"]))
    assert np.allclose(r["lse"][fin], lse_ref[fin], rtol=1e-14, atol=1e-13)


def test_large_scores_stay_finite_and_exact():
    # Scores multiplied by 40 (the stress case of section 16.2 "Measured"):
    # a max-free softmax overflows, the oracle must stay finite and exact.
    rng = np.random.default_rng(15)
    q, k, v = _rand((1, 2, 4, 8), rng, 3.0), _rand((1, 2, 6, 8), rng, 3.0), _rand((1, 2, 6, 8), rng)
    scale = 40.0 / math.sqrt(8)
    o_ref, lse_ref = brute_force(q, k, v, scale)
    r = oracle.attention(q, k, v, scale)
    assert np.all(np.isfinite(r["o"])) and np.all(np.isfinite(r["lse"]))
    with np.errstate(over="ignore", invalid="ignore"):
        s = scale * np.einsum("bhid,bhjd->bhij", q, k)
        naive = (np.exp(s) @ v) / np.exp(s).sum(-1, keepdims=True)
    assert not np.all(np.isfinite(naive))
    assert np.allclose(r["o"], o_ref, rtol=0, atol=1e-12)
    assert np.allclose(r["lse"], lse_ref, rtol=1e-14, atol=0)


# --------------------------------------------------------------- invariants
def test_gqa_equals_mha_on_repeated_heads():
    rng = np.random.default_rng(16)
    B, H, Hkv, Nq, Nk, d = 2, 8, 2, 5, 9, 4
    q, k, v = _rand((B, H, Nq, d), rng), _rand((B, Hkv, Nk, d), rng), _rand((B, Hkv, Nk, d), rng)
    hw = [0, 3, 0, 5, 2, 0, 1, 4]
    r = oracle.attention(q, k, v, 0.6, causal=True, head_window=hw, softcap=3.0)
    rep = H // Hkv
    kr, vr = np.repeat(k, rep, axis=1), np.repeat(v, rep, axis=1)
    r2 = oracle.attention(q, kr, vr, 0.6, causal=True, head_window=hw, softcap=3.0)
    assert np.allclose(r["o"], r2["o"], rtol=0, atol=0)
    assert np.array_equal(r["lse"], r2["lse"])
    # and each head really reads a different group: permuting groups changes it
    r3 = oracle.attention(q, k[:, ::-1], v[:, ::-1], 0.6, causal=True, head_window=hw, softcap=3.0)
    assert not np.allclose(r["o"], r3["o"])


@pytest.mark.parametrize("c", [5.0, 1000.0, -300.0])
def test_shift_invariance(c):
    # An extra dimension with q_e = c / scale, k_e = 1 adds c to every score:
    # O is unchanged and lse moves by exactly c.
    rng = np.random.default_rng(17)
    q, k, v = _rand((1, 2, 4, 3), rng), _rand((1, 2, 6, 3), rng), _rand((1, 2, 6, 3), rng)
    scale = 0.5
    r = oracle.attention(q, k, v, scale, causal=True)
    qe = np.concatenate([q, np.full((1, 2, 4, 1), c / scale)], axis=-1)
    ke = np.concatenate([k, np.ones((1, 2, 6, 1))], axis=-1)
    ve = np.concatenate([v, np.zeros((1, 2, 6, 1))], axis=-1)
    r2 = oracle.attention(qe, ke, ve, scale, causal=True)
    assert np.allclose(r2["o"][..., :3], r["o"], rtol=0, atol=1e-12)
    assert np.allclose(r2["lse"], r["lse"] + c, rtol=0, atol=1e-11 * max(1.0, abs(c)))


@pytest.mark.parametrize("tile", [1, 2, 3, 4, 8, 64])
@pytest.mark.parametrize("causal,W,cap", [(False, 0, 0.0), (True, 0, 0.0), (True, 5, 0.0), (True, 0, 4.0)])
def test_tiling_invariance(tile, causal, W, cap):
    # Streaming over key tiles of any size reproduces the direct result,
    # also with the causal mask applied by absolute position.
    rng = np.random.default_rng(18)
    q, k, v = _rand((1, 2, 13, 4), rng, 2.0), _rand((1, 2, 13, 4), rng, 2.0), _rand((1, 2, 13, 4), rng)
    d = oracle.attention(q, k, v, 0.7, causal=causal, window=W, softcap=cap)
    s = oracle.attention(q, k, v, 0.7, causal=causal, window=W, softcap=cap, tile=tile)
    assert np.allclose(s["o"], d["o"], rtol=0, atol=1e-13)
    assert np.allclose(s["lse"], d["lse"], rtol=1e-14, atol=0)


def test_scale_changes_the_output():
    rng = np.random.default_rng(19)
    q, k, v = (_rand((1, 1, 4, 16), rng) for _ in range(3))
    a = oracle.attention(q, k, v, 1.0 / (2.0 * 4.0))["o"]
    b = oracle.attention(q, k, v, 1.0 / (0.5 * 4.0))["o"]
    assert np.max(np.abs(a - b)) > 1e-4


def test_rows_subset_matches_full():
    rng = np.random.default_rng(20)
    q, k, v = _rand((2, 4, 6, 3), rng), _rand((2, 2, 7, 3), rng), _rand((2, 2, 7, 3), rng)
    full = oracle.attention(q, k, v, 0.9, causal=True, head_window=[0, 2, 3, 0])
    rows = np.array([0, 5, 17, 47, 30])
    sub = oracle.attention(q, k, v, 0.9, causal=True, head_window=[0, 2, 3, 0], rows=rows)
    assert np.array_equal(sub["o"], full["o"].reshape(-1, 3)[rows])
    assert np.array_equal(sub["lse"], full["lse"].reshape(-1)[rows])


def test_fa_seed_pattern_and_its_check():
    # The nx page's inputs: spot values, range, and its own check (streaming
    # equals direct to better than 1/1000) -- here far tighter.
    p = wl.fa_seed_pattern(64, 32)
    assert p["q"][0, 0, 0, 0] == np.float32(-6.0) / np.float32(13.0)
    assert p["k"][0, 0, 1, 2] == np.float32((5 + 4) % 11 - 5) / np.float32(11.0)
    assert p["v"][0, 0, 3, 1] == np.float32((9 + 1) % 9 - 4) / np.float32(9.0)
    for t in (p["q"], p["k"], p["v"]):
        assert t.min() >= -0.5 and t.max() <= 0.5
    scale = 1.0 / math.sqrt(32)
    d = oracle.attention(p["q"], p["k"], p["v"], scale)
    s = oracle.attention(p["q"], p["k"], p["v"], scale, tile=1)
    assert np.max(np.abs(d["o"] - s["o"])) < 1e-13


# ------------------------------------------------------------------- merge
def test_merge_exercise():
    g = golden("merge_exercise.json")
    o_part = np.array([[[1.0, 0.0], [0.0, 1.0]]])
    m_part = np.array([[g["m1"], g["m2"]]])
    l_part = np.array([[g["l1"], g["l2"]]])
    o, lse = oracle.combine(o_part, m_part, l_part)
    m = max(g["m1"], g["m2"])
    ell = math.exp(lse[0] - m)
    assert abs(ell - g["expected_l"]) < g["tolerance"]
    # Each block's output is weighted by its share of the merged sum, and the
    # shares add up to one.
    assert abs(o[0].sum() - 1.0) < 1e-15
    assert abs(o[0, 1] - g["l2"] / ell) < 1e-12


@pytest.mark.parametrize("S", [1, 2, 3, 4, 16])
@pytest.mark.parametrize("causal,W", [(False, 0), (True, 0), (True, 4)])
def test_split_invariance(S, causal, W):
    rng = np.random.default_rng(21)
    q, k, v = _rand((2, 4, 3, 5), rng, 1.5), _rand((2, 2, 19, 5), rng, 1.5), _rand((2, 2, 19, 5), rng)
    full = oracle.attention(q, k, v, 0.8, causal=causal, window=W)
    op, mp, lp = oracle.split_partials(q, k, v, 0.8, S, causal=causal, window=W)
    o, lse = oracle.combine(op, mp, lp)
    assert np.allclose(o, full["o"], rtol=0, atol=1e-13)
    assert np.allclose(lse, full["lse"], rtol=1e-14, atol=0)
    # Merging is insensitive to the order of the blocks.
    perm = rng.permutation(S)
    o2, lse2 = oracle.combine(op[..., perm, :], mp[..., perm], lp[..., perm])
    assert np.allclose(o2, o, rtol=0, atol=1e-13) and np.allclose(lse2, lse, rtol=1e-14, atol=0)


def test_split_partial_is_the_chunk_alone():
    # A partial is attention over its own chunk of keys only: with q = 0
    # its output is the chunk's mean value and l is its key count (m = 0).
    rng = np.random.default_rng(22)
    k, v = _rand((1, 1, 10, 3), rng), _rand((1, 1, 10, 3), rng)
    op, mp, lp = oracle.split_partials(np.zeros((1, 1, 1, 3)), k, v, 1.0, 3)
    for s, (lo, hi) in enumerate([(0, 4), (4, 8), (8, 10)]):
        assert np.allclose(op[0, 0, 0, s], v[0, 0, lo:hi].mean(axis=0), atol=1e-15)
        assert mp[0, 0, 0, s] == 0.0 and lp[0, 0, 0, s] == hi - lo


def test_merge_with_empty_partial_is_identity():
    rng = np.random.default_rng(23)
    o_part = np.stack([rng.standard_normal((4, 6)), np.zeros((4, 6))], axis=1)
    m_part = np.stack([rng.standard_normal(4), np.full(4, -np.inf)], axis=1)
    l_part = np.stack([rng.random(4) + 0.5, np.zeros(4)], axis=1)
    o, lse = oracle.combine(o_part, m_part, l_part)
    assert np.array_equal(o, o_part[:, 0])
    assert np.allclose(lse, m_part[:, 0] + np.log(l_part[:, 0]), rtol=1e-15, atol=0)
    o, lse = oracle.combine(np.zeros((2, 3, 4)), np.full((2, 3), -np.inf), np.zeros((2, 3)))
    assert np.all(o == 0) and np.all(np.isneginf(lse))


# Attention sinks with a sliding window (Transformers & Math 16.3 and 16.6):
# the first tokens stay visible to every windowed query.
SINK_CASES = [
    # B, H, Hkv, Nq, Nk, d, scale, head_window, softcap, sinks
    (1, 2, 1, 6, 9, 2, 1.0, [3, 2], 0.0, 2),
    (1, 1, 1, 5, 12, 3, 1.2, [2], 0.0, 4),
    (1, 2, 2, 4, 7, 2, 0.9, [1, 0], 2.0, 3),
    (1, 1, 1, 3, 3, 2, 1.0, [1], 0.0, 1),
]


@pytest.mark.parametrize("n", range(len(SINK_CASES)))
def test_sinks_match_decimal_brute_force(n):
    B, H, Hkv, Nq, Nk, d, scale, hw, cap, S = SINK_CASES[n]
    rng = np.random.default_rng(300 + n)
    q, k, v = _rand((B, H, Nq, d), rng), _rand((B, Hkv, Nk, d), rng), _rand((B, Hkv, Nk, d), rng)
    o_ref, lse_ref = brute_force(q, k, v, scale, True, hw, cap, sinks=S)
    r = oracle.attention(q, k, v, scale, causal=True, head_window=hw, softcap=cap, sinks=S)
    assert np.allclose(r["o"], o_ref, rtol=0, atol=1e-13)
    assert np.allclose(r["lse"], lse_ref, rtol=1e-14, atol=1e-13)


def test_sinks_covering_every_position_is_plain_causal():
    rng = np.random.default_rng(5)
    q, k, v = _rand((1, 2, 5, 3), rng), _rand((1, 2, 8, 3), rng), _rand((1, 2, 8, 3), rng)
    a = oracle.attention(q, k, v, 0.7, causal=True, window=2, sinks=8)
    b = oracle.attention(q, k, v, 0.7, causal=True)
    assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["lse"], b["lse"])


def test_sinks_need_no_window_to_matter():
    # without a window every causal key is visible anyway: sinks change nothing
    rng = np.random.default_rng(6)
    q, k, v = _rand((1, 1, 4, 3), rng), _rand((1, 1, 6, 3), rng), _rand((1, 1, 6, 3), rng)
    a = oracle.attention(q, k, v, 0.7, causal=True, sinks=3)
    b = oracle.attention(q, k, v, 0.7, causal=True)
    assert np.array_equal(a["o"], b["o"])


def test_uniform_scores_with_sinks_average_sink_and_window_values():
    # zero queries: every visible key has the same score, so O is the mean of
    # the visible values and lse the log of their count
    rng = np.random.default_rng(8)
    Nk, W, S = 20, 5, 4
    k, v = _rand((1, 1, Nk, 2), rng), _rand((1, 1, Nk, 2), rng)
    r = oracle.attention(np.zeros((1, 1, 1, 2)), k, v, 1.0, causal=True, window=W, sinks=S)
    keys = list(range(S)) + list(range(Nk - W, Nk))
    assert abs(r["lse"][0, 0, 0] - np.log(len(keys))) < 1e-14
    assert np.allclose(r["o"][0, 0, 0], v[0, 0, keys].mean(0), atol=1e-15)


def _ring_rows(pos, window, sinks):
    """Rows of a rolling cache (sinks rows first, then a ring of window slots)
    and the absolute position each holds after tokens 0..pos were written:
    token t < sinks goes to row t, token t >= sinks to row sinks + (t -
    sinks) % window, a later token replacing an earlier one."""
    rows = {}
    for t in range(pos + 1):
        rows[t if t < sinks else sinks + (t - sinks) % window] = t
    return rows


@pytest.mark.parametrize("pos,W,S", [(2, 4, 4), (6, 4, 4), (7, 4, 4), (30, 4, 4), (31, 5, 0), (9, 3, 2)])
def test_rolling_cache_equals_sink_window_attention(pos, W, S):
    # the decode query at position pos attending to every filled row of the
    # rolling cache sees exactly the sink + window keys of the full sequence
    rng = np.random.default_rng(pos * 10 + W)
    N, d = pos + 1, 3
    q, k, v = _rand((1, 2, 1, d), rng), _rand((1, 1, N, d), rng), _rand((1, 1, N, d), rng)
    rows = _ring_rows(pos, W, S)
    n = len(rows)
    assert sorted(rows) == list(range(n))  # filled rows form a prefix of the cache
    idx = [rows[r] for r in range(n)]
    ref = oracle.attention(q, k, v, 0.6, causal=True, window=W, sinks=S)
    got = oracle.attention(q, k[:, :, idx], v[:, :, idx], 0.6)
    assert np.allclose(got["o"], ref["o"], rtol=0, atol=1e-14)
    assert np.allclose(got["lse"], ref["lse"], rtol=0, atol=1e-14)
