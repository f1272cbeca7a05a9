"""Pins of the oracle's SwiGLU experts (O4), fp8 decode, combine (O5) and of the whole
layer: element loops, textbook special cases, OCP e4m3 values, identity experts and
the per-token formulation."""
import json
import math
import os

import numpy as np
import pytest

import moe_synth
import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden", "e4m3_values.json")


def test_swiglu_elementwise_loops():
    rng = np.random.default_rng(31)
    m, H, I = 3, 5, 4
    x = rng.standard_normal((m, H))
    wg, wu = rng.standard_normal((I, H)), rng.standard_normal((I, H))
    wd = rng.standard_normal((H, I))
    got = oracle.swiglu(x, wg, wu, wd)
    for r in range(m):
        h = []
        for i in range(I):
            a = sum(x[r, c] * wg[i, c] for c in range(H))
            b = sum(x[r, c] * wu[i, c] for c in range(H))
            h.append(a / (1.0 + math.exp(-a)) * b)
        for c in range(H):
            ref = sum(h[i] * wd[c, i] for i in range(I))
            assert abs(got[r, c] - ref) <= 1e-12 * (1 + abs(ref))


def test_swiglu_special_cases():
    rng = np.random.default_rng(32)
    x = rng.standard_normal((4, 6))
    wg, wu, wd = rng.standard_normal((3, 6)), rng.standard_normal((3, 6)), rng.standard_normal((6, 3))
    assert np.all(oracle.swiglu(x, np.zeros_like(wg), wu, wd) == 0)
    assert np.all(oracle.swiglu(x, wg, np.zeros_like(wu), wd) == 0)
    y1 = oracle.swiglu(x, wg, wu, wd)
    y2 = oracle.swiglu(x, wg, wu, 2.5 * wd)
    assert np.allclose(y2, 2.5 * y1, rtol=1e-13)
    # silu(z) -> z for large z, -> 0 for very negative z
    big = oracle.swiglu(np.array([[40.0]]), np.array([[1.0]]), np.array([[1.0]]), np.array([[1.0]]))
    assert abs(big[0, 0] - 1600.0) < 1e-9


def test_e4m3_decode_golden():
    g = json.load(open(GOLD))
    got = oracle.e4m3_decode(np.array(g["codes"], dtype=np.uint8))
    assert np.array_equal(got, np.array(g["values"]))
    assert np.isnan(oracle.e4m3_decode(np.array([0x7F, 0xFF], dtype=np.uint8))).all()


def test_e4m3_decode_matches_encoder_round_trip():
    # every finite code decodes to a value that the generator's encoder maps back to it
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    back = moe_synth.to_e4m3_codes(vals.astype(np.float32))
    zero = vals == 0
    assert np.array_equal(back[~zero], codes[~zero])
    assert np.all(np.diff(vals[:127]) > 0)          # monotone over the positive codes


def test_dequant_block_exact():
    rng = np.random.default_rng(33)
    w = (rng.standard_normal((256, 384)) * 0.02).astype(np.float32)
    q, s = moe_synth.block_quant_e4m3(w)
    d = oracle.dequant_block(q, s)
    assert d.shape == w.shape
    # per 128x128 block, |w - dequant| <= half an e4m3 step at that magnitude (3 mantissa bits)
    rel = np.abs(d - w) / np.maximum(np.abs(w), 2.0 ** -6 * np.repeat(np.repeat(s, 128, 0), 128, 1))
    assert rel.max() <= 2.0 ** -4 + 1e-12
    assert np.allclose(np.abs(d).reshape(2, 128, 3, 128).max(axis=(1, 3)), 448 * s, rtol=1e-6)


def test_combine_identity_experts():
    rng = np.random.default_rng(34)
    G, k, E, H = 40, 4, 16, 6
    x = rng.standard_normal((G, H)).astype(np.float32)
    logits = rng.standard_normal((G, E)).astype(np.float32)
    ids, w = oracle.select_grouped(logits, None, 4, 2, k, renormalize=True)
    plan = oracle.dispatch(ids, np.arange(E, dtype=np.int32)[:, None], np.ones(E, np.int32), 0, E, 8)
    xp = oracle.permute_rows(x, plan)
    out = oracle.combine(xp.astype(np.float64), plan, w, G)
    ref = (w.astype(np.float64).sum(axis=1))[:, None] * x
    assert np.allclose(out, ref, atol=1e-12)
    assert np.allclose(out, x, atol=1e-6)             # renormalised and all local -> x
    # only half the experts local: the weighted sum over the local ones
    plan2 = oracle.dispatch(ids, np.arange(E, dtype=np.int32)[:, None], np.ones(E, np.int32), 0, 8)
    out2 = oracle.combine(oracle.permute_rows(x, plan2).astype(np.float64), plan2, w, G, 2.0)
    wl = np.where(ids < 8, w, 0).astype(np.float64).sum(axis=1)
    assert np.allclose(out2, 2.0 * wl[:, None] * x, atol=1e-12)


def _small(cfg_name, tokens, H=256, I=128):
    from dataclasses import replace
    cfg = moe_synth.CONFIGS[cfg_name]
    return replace(cfg, num_tokens=tuple(tokens), static_bound=0, hidden=H, inter=I)


@pytest.mark.parametrize("name,tokens", [("cfg1", (64,)), ("cfg2", (9, 0, 17, 3)),
                                         ("cfg3", (5, 0, 7, 2)), ("cfg5", (6, 11))])
def test_layer_segment_form_equals_per_token_form(name, tokens):
    cfg = _small(name, tokens)
    inp = moe_synth.make_inputs(cfg)
    res = oracle.run_layer(inp, "max", align=4)
    cache = {}
    for g in range(res["layout"][1]):
        ref = oracle.token_output(inp, g, res["global_x"][g], res["ids"][g], res["weights"][g], cache)
        assert np.allclose(res["out"][g], ref, rtol=1e-10, atol=1e-12)


def test_layer_max_and_sum_modes_give_identical_replica_outputs():
    cfg = _small("cfg2", (9, 0, 17, 3))
    inp = moe_synth.make_inputs(cfg)
    a = oracle.run_layer(inp, "max")
    b = oracle.run_layer(inp, "sum")
    for ya, yb in zip(a["replicas_out"], b["replicas_out"]):
        assert np.array_equal(ya, yb)
    assert a["replicas_out"][1].shape[0] == 0        # idle replica gets zero rows


def test_replicated_slots_match_single_slot():
    # two slots holding one logical expert give the same output as a single slot would
    cfg = _small("cfg5", (13, 8))
    inp = moe_synth.make_inputs(cfg)
    res = oracle.run_layer(inp, "sum")
    # direct per-token evaluation with the logical expert's weights (first slot holding it)
    for g in range(res["layout"][1]):
        out = np.zeros(cfg.hidden)
        for j in range(cfg.top_k):
            lg = int(res["ids"][g, j])
            if lg < 0 or lg >= 12:
                continue
            slot = list(cfg.slot_logical).index(lg)
            x = oracle.as_f32(res["global_x"][g]).astype(np.float64)[None]
            out += float(res["weights"][g, j]) * oracle.swiglu(x, *oracle.expert_weights_f64(inp, slot))[0]
        assert np.allclose(res["out"][g], out, rtol=1e-10, atol=1e-12)


def test_zero_gate_weights_give_zero_output():
    cfg = _small("cfg3", (4, 6))
    inp = moe_synth.make_inputs(cfg)
    inp.w13[:, 0] = 0
    res = oracle.run_layer(inp, "sum")
    assert np.all(res["out"] == 0)


# ---------------------------------------------------------------- fp8 activations

def _finite_codes():
    return np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def test_e4m3_encode_round_trips_every_finite_code():
    codes = _finite_codes()
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_decode(codes)), codes)
    g = json.load(open(GOLD))
    assert np.array_equal(oracle.e4m3_encode(np.array(g["values"])), np.array(g["codes"], dtype=np.uint8))


def test_e4m3_encode_is_nearest_code_ties_to_even_brute_force():
    # every positive value's nearest code by exhaustive search over the 127 positive codes,
    # ties to the even code (the lower mantissa bit 0), at midpoints and just off them
    pos = np.arange(0, 0x7F, dtype=np.uint8)
    pv = oracle.e4m3_decode(pos)
    mids = (pv[:-1] + pv[1:]) / 2
    probes = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9), pv,
                             np.random.default_rng(1).uniform(0, 448, 5000)])
    for v in probes:
        d = np.abs(pv - v)
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else best[best % 2 == 0][0]
        assert oracle.e4m3_encode(np.array([v]))[0] == want, v
        assert oracle.e4m3_encode(np.array([-v]))[0] == (want | 0x80), v


def test_quant_group_closed_forms():
    rng = np.random.default_rng(5)
    # a group of e4m3 values times 2^j whose largest is 448 * 2^j: scale 2^j exactly, codes
    # returned unchanged, dequantisation exact
    codes = rng.integers(0, 0x7F, size=(6, 256)).astype(np.uint8) | (rng.integers(0, 2, size=(6, 256)) << 7).astype(np.uint8)
    codes[:, 5] = 0x7E
    codes[:, 130] = 0xFE
    j = rng.integers(-20, 20, size=(6, 1))
    x = (oracle.e4m3_decode(codes) * np.ldexp(1.0, j)).astype(np.float32)
    q, s = oracle.quant_group_e4m3(x)
    assert np.array_equal(s, np.repeat(np.ldexp(1.0, j), 2, axis=1).astype(np.float32))
    assert np.array_equal(q, codes)
    assert np.array_equal(oracle.dequant_group(q, s), x.astype(np.float64))
    # an all-zero group: scale 1, codes 0
    z = np.zeros((1, 128), dtype=np.float32)
    qz, sz = oracle.quant_group_e4m3(z)
    assert sz[0, 0] == 1.0 and not qz.any()


def test_quant_group_error_bound_and_amax_code():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((40, 384)) * np.exp(rng.uniform(-8, 8, (40, 1)))).astype(np.float32)
    q, s = oracle.quant_group_e4m3(x)
    # every group's largest magnitude lands on the largest code
    g = x.reshape(40, 3, 128)
    big = np.argmax(np.abs(g), axis=2)
    qg = q.reshape(40, 3, 128)
    assert np.all(np.take_along_axis(qg, big[..., None], axis=2)[..., 0] & 0x7F == 0x7E)
    # |x - dequant| is at most half a code step: 2^-4 |x| in the normal range of x / s,
    # 2^-10 s below it (subnormal step 2^-9), plus fp32 rounding of x / s
    d = oracle.dequant_group(q, s)
    ss = np.repeat(s.astype(np.float64), 128, axis=1)
    y = np.abs(x.astype(np.float64)) / ss
    bound = np.where(y >= 2.0 ** -6, 2.0 ** -4 * np.abs(x), 2.0 ** -10 * ss) * (1 + 2.0 ** -20)
    assert np.all(np.abs(d - x) <= bound)


def test_swiglu_e4m3_act_close_to_exact_and_exact_on_representable_input():
    rng = np.random.default_rng(7)
    H, I = 256, 128
    wg, wu = rng.standard_normal((I, H)) * 0.05, rng.standard_normal((I, H)) * 0.05
    wd = rng.standard_normal((H, I)) * 0.05
    x = rng.standard_normal((12, H)).astype(np.float32)
    y = oracle.swiglu_e4m3_act(x, wg, wu, wd)
    ref = oracle.swiglu(x.astype(np.float64), wg, wu, wd)
    assert oracle.rel_err(y, ref) < 0.1
    # with representable inputs and an identity down projection of a representable h the
    # fp8 path only rounds h to bf16 and to e4m3: compare against that composition
    # (e4m3 values of moderate size, each group's largest at 448, all times 2^-6)
    xs = (oracle.e4m3_decode(rng.integers(0x28, 0x48, size=(3, H)).astype(np.uint8))).astype(np.float32)
    xs[:, ::128] = 448.0
    xs *= np.float32(2.0 ** -6)
    h = oracle.bf16_rne(oracle.swiglu(xs.astype(np.float64), wg, wu, np.eye(I)))
    want = oracle.dequant_group(*oracle.quant_group_e4m3(h)) @ wd.T
    assert np.array_equal(oracle.swiglu_e4m3_act(xs, wg, wu, wd), want)
