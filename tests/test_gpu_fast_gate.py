"""The FAST gate (bf16 matrix-core logits, fp32 sums in tile order) against the oracle.

The products are the exact gate's, only their summation order differs, so the logits agree
to rounding.  Ids may then differ only at a near tie: with eps the largest logit difference
seen, a sigmoid key moves by at most eps/4 and a group score (two keys) by at most eps/2, so a
decision can flip only where the oracle's two candidates are within eps of each other.  Every
token whose ids differ must show such a gap (between the kept and dropped group scores, or
between adjacent keys among the k+1 best allowed experts).  Weights of agreeing tokens are
compared to tolerance."""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
from gpu_helpers import resized, say, to_np

pytestmark = pytest.mark.gpu


def _near_tie_grouped(logits, bias, n_group, topk_group, k, topn, eps):
    key = 1.0 / (1.0 + np.exp(-logits.astype(np.float64))) + (0.0 if bias is None else bias.astype(np.float64))
    G, E = key.shape
    per = E // n_group
    grp = np.sort(key.reshape(G, n_group, per), axis=2)[:, :, ::-1][:, :, :topn].sum(axis=2)
    gs = np.sort(grp, axis=1)[:, ::-1]
    gap_g = gs[:, topk_group - 1] - gs[:, topk_group] if topk_group < n_group else np.full(G, np.inf)
    order = np.argsort(-grp, axis=1, kind="stable")[:, :topk_group]
    allowed = np.zeros((G, n_group), dtype=bool)
    np.put_along_axis(allowed, order, True, axis=1)
    masked = np.where(np.repeat(allowed, per, axis=1), key, -np.inf)
    top = np.sort(masked, axis=1)[:, ::-1][:, :k + 1]
    gaps = top[:, :-1] - top[:, 1:]
    return (np.minimum(gap_g, np.nanmin(gaps, axis=1)) <= eps)


def _near_tie_softmax(logits, k, eps):
    top = np.sort(logits.astype(np.float64), axis=1)[:, ::-1][:, :k + 1]
    return np.min(top[:, :-1] - top[:, 1:], axis=1) <= eps


def _run_fast(inp, cfg):
    import combine_dp_gather_amd as m
    x = np.concatenate(inp.replicas)
    G = len(x)
    xd = torch.from_numpy(x).view(torch.bfloat16).cuda()
    wd = torch.from_numpy(inp.router_w).view(torch.bfloat16).cuda()
    bd = None if inp.bias is None else torch.from_numpy(inp.bias).cuda()
    rv = torch.ones(G, dtype=torch.int32, device="cuda")
    rc = m.make_route_cfg(cfg.route, cfg.num_experts, cfg.top_k, cfg.n_group, cfg.topk_group,
                          cfg.group_topn, cfg.renormalize, gate="fast")
    lg = torch.empty(G, cfg.num_experts, device="cuda")
    ids = torch.empty(G, cfg.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(G, cfg.top_k, device="cuda")
    m.moe_route(xd, rv, wd, bd, rc, lg, ids, w)
    torch.cuda.synchronize()
    return x, to_np(lg), to_np(ids), to_np(w)


@pytest.mark.parametrize("name", ["cfg4", "cfg2"])
def test_fast_gate_near_tie_audit(name):
    base = moe_synth.CONFIGS[name]
    cfg = resized("cfg4", (1500, 1300, 1296)) if name == "cfg4" else base
    say(f"[fast gate] {cfg.name} tokens={sum(cfg.num_tokens)} H={cfg.hidden} E={cfg.num_experts}")
    inp = moe_synth.make_inputs(cfg, with_experts=False)
    x, lg, ids, w = _run_fast(inp, cfg)
    G = len(x)
    ref_l, ref_ids, ref_w = oracle.route(cfg, x, np.ones(G, np.int32), inp.router_w, inp.bias)
    diff = np.abs(lg.astype(np.float64) - ref_l)
    eps = float(diff.max())
    say(f"  max |logit diff| {eps:.3e} (max |logit| {np.abs(ref_l).max():.3e})")
    assert eps <= 1e-4 * max(float(np.abs(ref_l).max()), 1.0)
    bad = np.any(ids != ref_ids, axis=1)
    if cfg.route == "grouped":
        tie = _near_tie_grouped(ref_l, inp.bias, cfg.n_group, cfg.topk_group, cfg.top_k, cfg.group_topn, eps)
    else:
        tie = _near_tie_softmax(ref_l, cfg.top_k, eps)
    say(f"  tokens with different ids: {int(bad.sum())}; oracle near ties within eps: {int(tie.sum())}")
    assert not np.any(bad & ~tie), np.nonzero(bad & ~tie)[0][:10]
    ok = ~bad
    assert oracle.rel_err(w[ok], ref_w[ok]) < 1e-4


def test_fast_mode_small_batch_is_exact():
    """A decode-sized batch in FAST mode runs the exact single-chain gate: logits and ids
    equal the oracle's bit for bit."""
    import combine_dp_gather_amd as m
    cfg = moe_synth.CONFIGS["cfg3"]
    inp = moe_synth.make_inputs(cfg, with_experts=False)
    x = np.concatenate(inp.replicas)
    G = len(x)
    rc = m.make_route_cfg(cfg.route, cfg.num_experts, cfg.top_k, cfg.n_group, cfg.topk_group,
                          cfg.group_topn, cfg.renormalize, gate="fast")
    lg = torch.empty(G, cfg.num_experts, device="cuda")
    ids = torch.empty(G, cfg.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(G, cfg.top_k, device="cuda")
    m.moe_route(torch.from_numpy(x).view(torch.bfloat16).cuda(), torch.ones(G, dtype=torch.int32, device="cuda"),
                torch.from_numpy(inp.router_w).view(torch.bfloat16).cuda(), torch.from_numpy(inp.bias).cuda(), rc,
                lg, ids, w)
    torch.cuda.synchronize()
    ref_l, ref_ids, ref_w = oracle.route(cfg, x, np.ones(G, np.int32), inp.router_w, inp.bias)
    assert np.array_equal(to_np(lg).view(np.uint32), ref_l.view(np.uint32))
    assert np.array_equal(to_np(ids), ref_ids)


# FAST mode runs its own kernels once its 128-row x 256-expert tiles cover half the CUs
@pytest.mark.parametrize("G,H,E", [(16384, 7168, 256), (8200, 2048, 320), (16400, 512, 256)])
def test_fast_dma_kernel_equals_register_staged_kernel(G, H, E):
    """FAST mode has two kernels with one tile and one K order: LDS-DMA staging for aligned
    rows with H a multiple of 64, register staging otherwise.  The same rows run once from an
    aligned buffer and once from a buffer offset by 2 bytes (which forces register staging):
    the logits must agree bit for bit, invalid rows must be 0, and a ragged last tile (G not a
    multiple of 128, E not a multiple of 256) must be covered."""
    import combine_dp_gather_amd as m
    rng = np.random.default_rng(7)
    x = torch.from_numpy(rng.standard_normal((G, H), dtype=np.float32)).to(torch.bfloat16).cuda()
    wr = torch.from_numpy((0.02 * rng.standard_normal((E, H))).astype(np.float32)).to(torch.bfloat16).cuda()
    rv = torch.from_numpy((rng.random(G) > 0.1).astype(np.int32)).cuda()
    rc = m.make_route_cfg("softmax", E, 8, 1, 1, 1, True, gate="fast")
    outs = []
    for shifted in (False, True):
        if shifted:
            buf = torch.empty(G * H + 1, dtype=torch.bfloat16, device="cuda")
            xs = buf[1:].view(G, H)
            xs.copy_(x)
        else:
            xs = x
        lg = torch.full((G, E), float("nan"), device="cuda")
        ids = torch.empty(G, 8, dtype=torch.int32, device="cuda")
        w = torch.empty(G, 8, device="cuda")
        m.moe_route(xs, rv, wr, None, rc, lg, ids, w)
        torch.cuda.synchronize()
        outs.append(to_np(lg))
    say(f"[fast] G={G} H={H} E={E}: DMA and register-staged FAST logits compared")
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    invalid = to_np(rv) == 0
    assert np.all(outs[0][invalid] == 0.0)
    ref = x.float() @ wr.float().t()
    d = (torch.from_numpy(outs[0]).cuda() - ref).abs()[torch.from_numpy(~invalid).cuda()]
    assert float(d.max()) < 1e-3 * float(ref.abs().max())
