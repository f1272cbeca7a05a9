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
