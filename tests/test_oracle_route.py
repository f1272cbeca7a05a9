"""Pins of the oracle's routing (O2): exact gate logits against exact rational
arithmetic, the defined exp against the platform exp, and both selection rules
against exhaustive subset enumeration and a stable library sort."""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import moe_synth
import oracle


# ---------------------------------------------------------------- exact fp32 rounding

def round_f32(v: Fraction) -> float:
    """Round an exact rational to the nearest fp32 (ties to even), as a Python float."""
    if v == 0:
        return 0.0
    s = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                     # subnormal spacing below 2^-126
    q = a / (Fraction(2) ** (e - 23))   # scaled so one fp32 ulp is 1
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return s * float(Fraction(fl) * Fraction(2) ** (e - 23))


def fma_chain(x, w):
    """One fp32 fma chain over h in ascending order from +0, in exact rational arithmetic
    rounded to fp32 at every step."""
    acc = 0.0
    for a, b in zip(x, w):
        acc = round_f32(Fraction(float(a)) * Fraction(float(b)) + Fraction(acc))
    return acc


def test_round_f32_matches_numpy_cast():
    rng = np.random.default_rng(3)
    for v in rng.standard_normal(300) * 10.0 ** rng.integers(-30, 30, 300):
        assert round_f32(Fraction(float(v))) == float(np.float32(v))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gate_logits_bitwise_vs_exact_fma(dtype):
    rng = np.random.default_rng(1)
    G, E, H = 4, 5, 300
    x = rng.standard_normal((G, H)).astype(np.float32)
    w = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    if dtype == "bf16":
        x, w = moe_synth.to_bf16_bits(x), moe_synth.to_bf16_bits(w)
    got = oracle.gate_logits(x, w)
    xf, wf = oracle.as_f32(x), oracle.as_f32(w)
    for g in range(G):
        for e in range(E):
            assert got[g, e] == np.float32(fma_chain(xf[g], wf[e])), (g, e)


def test_gate_logits_bf16_equals_plain_f32_adds():
    # bf16 x bf16 products are exact in fp32, so the fma chain is a chain of IEEE fp32 adds
    # of the exact products in ascending h, which numpy's float32 add computes independently
    rng = np.random.default_rng(2)
    H = 300
    x = moe_synth.to_bf16_bits(rng.standard_normal((4, H)).astype(np.float32))
    w = moe_synth.to_bf16_bits((rng.standard_normal((9, H)) * 0.02).astype(np.float32))
    xf, wf = oracle.as_f32(x), oracle.as_f32(w)
    acc = np.zeros((4, 9), dtype=np.float32)
    for h in range(H):
        acc = acc + (xf[:, h:h + 1] * wf[None, :, h])
    assert np.array_equal(oracle.gate_logits(x, w), acc)


def test_gate_logits_order_closed_form():
    # products 2^24, 1, -2^24 in this h order: ascending from +0 gives 2^24 (2^24 + 1 is a
    # tie that rounds to the even 2^24), then 0.  Any other order, a pairwise tree or the
    # exact sum gives 1: the ascending single chain is the only reading that yields 0.
    w = np.ones((1, 3), dtype=np.float32)
    x = np.array([[2.0 ** 24, 1.0, -(2.0 ** 24)]], dtype=np.float32)
    assert oracle.gate_logits(x, w)[0, 0] == 0.0
    # reversed h order: -2^24 + 1 is exact, + 2^24 gives 1
    assert oracle.gate_logits(x[:, ::-1].copy(), w)[0, 0] == 1.0
    # the same three products at h = 127, 128, 129 among zero products: 128-wide chunk
    # sums would give 2^24 + (1 - 2^24) = 1, the single chain still 0
    xz = np.zeros((1, 203), dtype=np.float32)
    xz[0, 127:130] = x[0]
    assert oracle.gate_logits(xz, np.ones((1, 203), dtype=np.float32))[0, 0] == 0.0


def test_gate_is_one_chain_not_chunked():
    # a chunked reading (128-wide fma chains, chunk sums added left to right) differs from
    # the single chain on ordinary inputs, so the pins above would catch an oracle that
    # chunked h
    rng = np.random.default_rng(5)
    x = moe_synth.to_bf16_bits(rng.standard_normal((64, 1024)).astype(np.float32))
    w = moe_synth.to_bf16_bits((rng.standard_normal((8, 1024)) * 0.02).astype(np.float32))
    xf, wf = oracle.as_f32(x), oracle.as_f32(w)
    total = np.zeros((64, 8), dtype=np.float32)
    for c0 in range(0, 1024, 128):
        part = np.zeros((64, 8), dtype=np.float32)
        for h in range(c0, c0 + 128):
            part = part + (xf[:, h:h + 1] * wf[None, :, h])
        total = total + part
    got = oracle.gate_logits(x, w)
    assert not np.array_equal(got, total)
    assert np.count_nonzero(got != total) > 8


def test_gate_logits_one_hot_and_pad_rows():
    rng = np.random.default_rng(4)
    w = rng.standard_normal((7, 16)).astype(np.float32)
    x = np.zeros((3, 16), dtype=np.float32)
    x[0, 5] = 1.0
    x[1, 9] = 1.0
    x[2, 3] = 1.0
    got = oracle.gate_logits(x, w, row_valid=np.array([1, 1, 0], dtype=np.int32))
    assert np.array_equal(got[0], w[:, 5]) and np.array_equal(got[1], w[:, 9])
    assert np.all(got[2] == 0)


# ---------------------------------------------------------------- defined exp / sigmoid

def test_exp_defined_close_to_platform_exp():
    xs = np.concatenate([np.linspace(-40, 40, 4001), [-700.0, -300.5, 0.3466, -0.3466, 88.7, 700.0]])
    for v in xs:
        ref = math.exp(v)
        got = oracle.exp_defined(v)
        assert abs(got - ref) <= 2 * math.ulp(ref), v
    assert oracle.exp_defined(0.0) == 1.0
    assert oracle.exp_defined(1000.0) == math.inf
    assert oracle.exp_defined(-1000.0) == 0.0


def test_sigmoid_defined():
    assert oracle.sigmoid_defined(0.0) == 0.5
    prev = -1.0
    for v in np.linspace(-30, 30, 2001):
        s = oracle.sigmoid_defined(v)
        assert abs(s - 1.0 / (1.0 + math.exp(-v))) <= 4e-16
        assert s >= prev
        prev = s


# ---------------------------------------------------------------- softmax top-k

def _best_subset(keys, k, allowed=None):
    idx = [i for i in range(len(keys)) if allowed is None or allowed[i]]
    return max(itertools.combinations(idx, k), key=lambda c: (sum(keys[i] for i in c), [-i for i in c]))


def test_softmax_topk_exhaustive():
    rng = np.random.default_rng(8)
    logits = rng.standard_normal((200, 8)).astype(np.float32)
    ids, w = oracle.select_softmax(logits, 2, renormalize=False)
    for g in range(200):
        best = _best_subset([float(v) for v in logits[g]], 2)
        assert set(ids[g]) == set(best)
        assert logits[g, ids[g, 0]] >= logits[g, ids[g, 1]]
        p = np.exp(logits[g].astype(np.float64) - logits[g].max())
        p /= p.sum()
        assert np.allclose(w[g], p[ids[g]], rtol=1e-6, atol=0)


def test_softmax_topk_matches_stable_argsort_and_renorm():
    rng = np.random.default_rng(9)
    logits = rng.standard_normal((300, 64)).astype(np.float32)
    logits[:, 10] = logits[:, 3]             # exact ties
    ids, w = oracle.select_softmax(logits, 6, renormalize=True)
    ref = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")[:, :6]
    assert np.array_equal(ids, ref)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)


def test_softmax_ties_lower_id_first():
    logits = np.full((1, 8), 2.0, dtype=np.float32)
    ids, w = oracle.select_softmax(logits, 3)
    assert list(ids[0]) == [0, 1, 2]
    assert np.allclose(w, 1.0 / 8)


def test_pad_rows_masked():
    logits = np.ones((3, 16), dtype=np.float32)
    rv = np.array([1, 0, 1], dtype=np.int32)
    ids, w = oracle.select_softmax(logits, 2, row_valid=rv)
    assert list(ids[1]) == [-1, -1] and np.all(w[1] == 0)
    ids, w = oracle.select_grouped(logits, None, 4, 2, 2, row_valid=rv)
    assert list(ids[1]) == [-1, -1] and np.all(w[1] == 0)


# ---------------------------------------------------------------- grouped sigmoid top-k

def _grouped_brute(l, b, n_group, topk_group, k, topn):
    E = len(l)
    per = E // n_group
    s = [1.0 / (1.0 + math.exp(-float(v))) for v in l]
    key = [s[e] + float(b[e]) for e in range(E)]
    gs = []
    for q in range(n_group):
        ks = sorted(key[q * per:(q + 1) * per], reverse=True)[:topn]
        gs.append(sum(ks))
    groups = _best_subset(gs, topk_group)
    allowed = [e // per in groups for e in range(E)]
    chosen = _best_subset(key, k, allowed)
    order = sorted(chosen, key=lambda e: (-key[e], e))
    tot = sum(s[e] for e in order)
    return order, [s[e] / tot for e in order]


def test_grouped_exhaustive_tiny():
    rng = np.random.default_rng(10)
    G, E = 300, 16
    logits = rng.standard_normal((G, E)).astype(np.float32)
    bias = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    ids, w = oracle.select_grouped(logits, bias, n_group=4, topk_group=2, k=4, renormalize=True)
    for g in range(G):
        order, ww = _grouped_brute(logits[g], bias, 4, 2, 4, 2)
        assert list(ids[g]) == order, g
        assert np.allclose(w[g], ww, rtol=1e-6)


def test_grouped_weights_exclude_bias_and_renorm_flag():
    rng = np.random.default_rng(12)
    logits = rng.standard_normal((50, 32)).astype(np.float32)
    bias = rng.uniform(-0.5, 0.5, 32).astype(np.float32)
    ids, w = oracle.select_grouped(logits, bias, 4, 2, 4, renormalize=False)
    sig = 1.0 / (1.0 + np.exp(-logits.astype(np.float64)))
    assert np.allclose(w, np.take_along_axis(sig, ids, 1), rtol=1e-6)


def test_grouped_group_tie_break_lower_group():
    # every key equal: groups 0,1 win the group stage, experts 0..3 win the expert stage
    logits = np.zeros((1, 16), dtype=np.float32)
    ids, w = oracle.select_grouped(logits, None, 4, 2, 4)
    assert list(ids[0]) == [0, 1, 2, 3]
    assert np.allclose(w, 0.25)


def test_grouped_bias_steers_selection():
    # a large bias on one group pulls every token into it
    logits = np.random.default_rng(13).standard_normal((64, 16)).astype(np.float32)
    bias = np.zeros(16, dtype=np.float32)
    bias[12:16] = 5.0
    ids, _ = oracle.select_grouped(logits, bias, 4, 1, 4)
    assert np.all(np.sort(ids, axis=1) == np.arange(12, 16))


def test_fake_uniform_logits_balanced():
    # ep_dispatch_algorithm "fake": logits U(5,10), bias zeroed -> near-uniform load
    G, E, k = 4096, 256, 8
    logits = moe_synth.fake_uniform_logits(0, G, E)
    ids, _ = oracle.select_grouped(logits, np.zeros(E, np.float32), 8, 4, k)
    hist = np.bincount(ids.ravel(), minlength=E)
    mean = G * k / E
    assert hist.min() > 0.6 * mean and hist.max() < 1.4 * mean
    bal = (hist.mean() + 1e-5) / (hist.max() + 1e-5)
    assert bal > 0.7


def test_zipf_bias_gives_slope_near_minus_1_2():
    # skewed-load workload: popularity p_e ~ (e+1)^-1.2 imposed through the router bias
    # (bias = beta * ln(p_e / p_0)); with beta = 0.12 the realised rank-frequency slope of
    # the routed ids over the 64 most used experts is -1.2 within 0.1 (4096 tokens)
    from dataclasses import replace
    cfg = moe_synth.CONFIGS["cfg5"]
    small = replace(cfg, num_tokens=(2048, 2048))
    inp = moe_synth.make_inputs(small, with_experts=False)
    x = np.concatenate(inp.replicas)
    _, ids, _ = oracle.route(small, x, np.ones(len(x), np.int32), inp.router_w, inp.bias)
    freq = np.sort(np.bincount(ids.ravel(), minlength=cfg.num_experts))[::-1][:64].astype(np.float64)
    slope = np.polyfit(np.log(np.arange(1, 65)), np.log(freq), 1)[0]
    assert -1.3 < slope < -1.1, slope
