"""Full-size parity at the two prefill workloads, in the launch configuration bench.py times
(gather mode "sum", no alignment, default capacity):

  prefill bf16  8 DP replicas x 4096 tokens, H=7168, E=256 grouped top-8, 16 local experts, I=2048
  prefill fp8   8 x 2048 tokens, Zipf-biased routing, 16 slots holding 12 logical experts,
                e4m3 weights with 128x128 block scales, with bf16 activations (the default)
                and with e4m3 activations quantised per 1x128 group (the oracle then
                quantises them too: codes bitwise)

Every integer and every copied byte is compared bit for bit against the oracle over the
whole batch: the gathered rows, all G x E gate logits, all expert ids, the whole dispatch
plan, the permuted rows and the scattered replica slices.  The floating-point outputs are
compared on every row:
  - y_perm, every routed row, against the oracle's float64 experts: per-row relative error
    (a row's largest deviation over its largest reference value) within the bar;
  - combine in isolation: the oracle's float64 combine of the device's own y_perm and
    weights, against the device's out, element by element within one bf16 ulp of the
    reference plus the fp32 accumulation bound 2 (k + 1) 2^-24 sum_j |w_j y_j|;
  - out, every row, against the oracle's whole layer: per-row relative error within the bar.
"""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
from gpu_helpers import build_layer, check_combine_bound, copy_path_rows, replicas_to_device, say, to_np, tol_for

pytestmark = pytest.mark.gpu


def _expert_rows(inp, xp, plan):
    """The oracle's y_perm (float64) on every routed row, one slot at a time."""
    R = plan["num_rows"]
    y = np.zeros((R, inp.cfg.hidden), dtype=np.float64)
    seg, counts = plan["seg_offsets"], plan["counts"]
    for e in range(len(counts)):
        a, n = int(seg[e]), int(counts[e])
        if n:
            y[a:a + n] = oracle.swiglu(oracle.as_f32(xp[a:a + n]).astype(np.float64),
                                       *oracle.expert_weights_f64(inp, e))
    return y


def _check_expert_rows(y_dev, y_ref, plan, tol, label):
    seg, counts = plan["seg_offsets"], plan["counts"]
    worst = 0.0
    for e in range(len(counts)):
        a, n = int(seg[e]), int(counts[e])
        if n:
            worst = max(worst, oracle.row_rel_err(oracle.as_f32(y_dev[a:a + n]), y_ref[a:a + n]))
    say(f"  {label}: y_perm, all {int(np.sum(counts))} rows, largest per-row error {worst:.3e}")
    assert worst < tol


def _check_combine_bound(out_dev, y_dev, w_dev, pair_row, k, label):
    worst = check_combine_bound(out_dev, y_dev, w_dev, pair_row, k)
    say(f"  {label}: combine of the device's y_perm, all {len(pair_row) // k} rows: "
        f"largest deviation {worst:.2f} of the bound")


def _check_out_rows(out_dev, out_ref, tol, label):
    err = oracle.row_rel_err(oracle.as_f32(out_dev), out_ref)
    say(f"  {label}: out, all {len(out_ref)} rows, largest per-row error {err:.3e}")
    assert err < tol


@pytest.mark.parametrize("name", ["cfg4", "cfg5"])
def test_prefill_fullsize(name):
    cfg = moe_synth.CONFIGS[name]
    say(f"[fullsize] {name}: tokens={cfg.num_tokens} H={cfg.hidden} I={cfg.inter} E={cfg.num_experts} "
        f"slots={cfg.num_local} weights={cfg.weight_format}")
    inp = moe_synth.make_inputs(cfg)
    layer = build_layer(inp, "sum")
    layer.forward(replicas_to_device(inp))
    torch.cuda.synchronize()
    say("  gpu forward done")
    k, H = cfg.top_k, cfg.hidden

    # S1 gather
    layout = oracle.gather_layout(cfg.num_tokens, "sum", static_bound=cfg.static_bound)
    G = layout[1]
    assert layer.G == G and layer.offsets == layout[2]
    gx, valid = oracle.gather(layout, inp.replicas, H, np.uint16)
    assert np.array_equal(to_np(layer.global_x), gx)
    assert np.array_equal(to_np(layer.row_valid)[:G], valid)

    # S2 route: every logit and id
    logits, ids, w = oracle.route(cfg, gx, valid, inp.router_w, inp.bias)
    say("  oracle route done")
    assert np.array_equal(to_np(layer.logits)[:G].view(np.uint32), logits.view(np.uint32))
    assert np.array_equal(to_np(layer.topk_ids)[:G], ids)
    assert oracle.rel_err(to_np(layer.topk_w)[:G], w) < 1e-5

    # S3 dispatch: the whole plan and every permuted row
    plan = oracle.dispatch(ids, inp.phys_of, inp.n_rep, cfg.first_local, cfg.num_local, 1, None)
    gp = layer.plan
    assert np.array_equal(to_np(gp.counts), plan["counts"])
    assert np.array_equal(to_np(gp.seg_offsets), plan["seg_offsets"])
    assert int(to_np(gp.num_rows)[0]) == plan["num_rows"]
    assert int(to_np(gp.error_flag)[0]) == 0 == plan["error_flag"]
    R = plan["num_rows"]
    assert np.array_equal(to_np(gp.sorted_pair)[:R], plan["sorted_pair"])
    assert np.array_equal(to_np(gp.pair_row)[:G * k], plan["pair_row"])
    # the layer's up GEMM gathers its rows from global_x; the permuted copy runs beside it, is
    # held to the oracle, and the copy path's h to the gathered one, every routed row bitwise
    xp = oracle.permute_rows(gx, plan)
    xp_dev, h_copy = copy_path_rows(layer)
    assert np.array_equal(to_np(xp_dev)[:R], xp)
    real = np.zeros(R, dtype=bool)
    for e in range(cfg.num_local):
        a = int(plan["seg_offsets"][e])
        real[a:a + int(plan["counts"][e])] = True
    assert np.array_equal(to_np(layer.h)[:R][real], to_np(h_copy)[:R][real])
    del h_copy
    say(f"  plan and permuted rows bitwise (R={R}); gathered h equals the copy path's")

    tol = tol_for(cfg)
    y_ref = _expert_rows(inp, xp, plan)
    say("  oracle experts done")
    _check_expert_rows(to_np(layer.y_perm)[:R], y_ref, plan, tol, "bf16 activations")
    _check_combine_bound(to_np(layer.out), to_np(layer.y_perm)[:R], to_np(layer.topk_w)[:G],
                         plan["pair_row"], k, "bf16 activations")
    out_ref = oracle.combine(y_ref, plan, w, G)
    _check_out_rows(to_np(layer.out), out_ref, tol, "bf16 activations")

    # S6 scatter: each replica slice is a copy of the device's own combined rows
    offs = layout[2]
    out_np = to_np(layer.out)
    for i, y in enumerate(layer.replicas_out):
        a, n = offs[i], cfg.num_tokens[i]
        assert np.array_equal(to_np(y), out_np[a:a + n])
    # the fused exit (what bench.py's step runs): the same bits in every replica's buffer
    fresh = [torch.full_like(y, 5.0) for y in layer.replicas_out]
    layer.combine_scatter(fresh)
    torch.cuda.synchronize()
    for y, f in zip(layer.replicas_out, fresh):
        assert torch.equal(y.view(torch.int16), f.view(torch.int16))
    del fresh
    say("  fused exit: every replica row bitwise equal to combine, then scatter")

    if cfg.weight_format != "fp8_block":
        return
    # the same batch with e4m3 activations (1x128 groups, 56 groups along H=7168, 16 along
    # I=2048) on the fp8 matrix cores.  The oracle quantises the activations the same way, so
    # every code of x_perm is compared bit for bit.  The codes of h can differ by one step
    # where the device's fp32-accumulated h and the oracle's float64 one round to different
    # bf16 values next to a code boundary, and one such step on a large element moves its row
    # by ~1.4e-2, so the outputs are held to the fp8 bar.  What the quantisation itself costs
    # against the unquantised experts is reported
    del layer, out_np
    torch.cuda.empty_cache()
    # (xp_dev, the copied rows, is kept for the quantisation check below)
    layer = build_layer(inp, "sum", fp8_act="e4m3")
    layer.forward(replicas_to_device(inp))
    torch.cuda.synchronize()
    assert np.array_equal(to_np(layer.plan.sorted_pair)[:R], plan["sorted_pair"])
    h_copy = copy_path_rows(layer)[1]  # the quantiser reads gathered rows: the same codes
    assert np.array_equal(to_np(layer.h)[:R][real], to_np(h_copy)[:R][real])
    del h_copy
    import combine_dp_gather_amd as m
    q = torch.empty((R, H), dtype=torch.uint8, device="cuda")
    st = torch.empty((H // 128, R), dtype=torch.float32, device="cuda")
    m.moe_quant_act_fp8(xp_dev[:R], layer.plan.num_rows, q, st)
    torch.cuda.synchronize()
    rq, rs = oracle.quant_group_e4m3(xp)
    assert np.array_equal(to_np(q), rq)
    assert np.array_equal(to_np(st).view(np.uint32), rs.T.view(np.uint32))
    say(f"  e4m3 activations: all {R} x {H} codes and scales of x_perm bitwise")
    seg, counts = plan["seg_offsets"], plan["counts"]
    yq = np.zeros_like(y_ref)
    for e in range(len(counts)):
        a, n = int(seg[e]), int(counts[e])
        if n:
            yq[a:a + n] = oracle.swiglu_e4m3_act(xp[a:a + n], *oracle.expert_weights_f64(inp, e))
    say(f"  e4m3 activations: quantisation alone against the unquantised experts: rel err "
        f"{oracle.rel_err(yq, y_ref):.3e}, largest per-row {oracle.row_rel_err(yq, y_ref):.3e}")
    _check_expert_rows(to_np(layer.y_perm)[:R], yq, plan, tol, "e4m3 activations")
    _check_combine_bound(to_np(layer.out), to_np(layer.y_perm)[:R], to_np(layer.topk_w)[:G],
                         plan["pair_row"], k, "e4m3 activations")
    _check_out_rows(to_np(layer.out), oracle.combine(yq, plan, w, G), tol, "e4m3 activations")
