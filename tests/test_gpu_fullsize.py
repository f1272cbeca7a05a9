"""Full-size parity at the two prefill workloads, in the launch configuration bench.py times
(gather mode "sum", no alignment, default capacity):

  prefill bf16  8 DP replicas x 4096 tokens, H=7168, E=256 grouped top-8, 16 local experts, I=2048
  prefill fp8   8 x 2048 tokens, Zipf-biased routing, 16 slots holding 12 logical experts,
                e4m3 weights with 128x128 block scales

Every integer and every copied byte is compared bit for bit against the oracle over the
whole batch: the gathered rows, all G x E gate logits, all expert ids, the whole dispatch
plan, the permuted rows and the scattered replica slices.  The floating-point expert and
combine outputs are compared on sampled rows that the oracle computes one at a time
(every segment's first and last row, every replica's first and last token, plus seeded
random picks)."""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
from gpu_helpers import build_layer, replicas_to_device, say, to_np, tol_for

pytestmark = pytest.mark.gpu


def _sample_segment_rows(rng, seg, counts, n_random):
    rows = []
    for e in range(len(counts)):
        if counts[e]:
            rows += [int(seg[e]), int(seg[e]) + int(counts[e]) - 1]
    real = np.concatenate([np.arange(seg[e], seg[e] + counts[e]) for e in range(len(counts))])
    rows += [int(v) for v in rng.choice(real, size=min(n_random, real.size), replace=False)]
    return sorted(set(rows))


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
    xp = oracle.permute_rows(gx, plan)
    assert np.array_equal(to_np(layer.x_perm)[:R], xp)
    say(f"  plan and permuted rows bitwise (R={R})")

    rng = np.random.default_rng(1234)
    tol = tol_for(cfg)
    cache = {}

    # S4 experts on sampled rows of every segment
    rows = _sample_segment_rows(rng, plan["seg_offsets"], plan["counts"], 24)
    y_gpu = oracle.as_f32(to_np(layer.y_perm)[rows]).astype(np.float64)
    y_ref = np.empty_like(y_gpu)
    for i, r in enumerate(rows):
        e = int(np.searchsorted(plan["seg_offsets"], r, side="right") - 1)
        if e not in cache:
            cache[e] = oracle.expert_weights_f64(inp, e)
        y_ref[i] = oracle.swiglu(oracle.as_f32(xp[r:r + 1]).astype(np.float64), *cache[e])[0]
    err = oracle.rel_err(y_gpu, y_ref)
    say(f"  y_perm on {len(rows)} sampled rows: rel err {err:.3e}")
    assert err < tol

    # S5 combine on sampled tokens (replica edges + random), computed directly per token
    offs = layout[2]
    toks = set()
    for i, n in enumerate(cfg.num_tokens):
        if n:
            toks |= {offs[i], offs[i] + n - 1}
    toks |= {int(v) for v in rng.choice(G, size=24, replace=False)}
    toks = sorted(toks)
    out_gpu = oracle.as_f32(to_np(layer.out)[toks]).astype(np.float64)
    out_ref = np.stack([oracle.token_output(inp, g, gx[g], ids[g], w[g], cache) for g in toks])
    err = oracle.rel_err(out_gpu, out_ref)
    say(f"  out on {len(toks)} sampled tokens: rel err {err:.3e}")
    assert err < tol

    # S6 scatter: each replica slice is a copy of the device's own combined rows
    out_np = to_np(layer.out)
    for i, y in enumerate(layer.replicas_out):
        a, n = offs[i], cfg.num_tokens[i]
        assert np.array_equal(to_np(y), out_np[a:a + n])
