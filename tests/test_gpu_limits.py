"""The path at the limits the C ABI declares: 1024 logical experts, top-32, 64 groups with
group top-4, 1024 local slots, and up to 256 DP replicas (several launches of the 32-replica
gather / scatter / entry batches), each against the oracle at the usual bar."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import moe_synth
import oracle
from gpu_helpers import say, to_np

pytestmark = pytest.mark.gpu


def _select(m, lg, cfg, bias=None, rv=None):
    G, E = lg.shape
    ids = torch.empty((G, cfg.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((G, cfg.top_k), dtype=torch.float32, device="cuda")
    m.moe_route_from_logits(torch.from_numpy(lg).cuda(), None if rv is None else torch.from_numpy(rv).cuda(),
                            None if bias is None else torch.from_numpy(bias).cuda(), cfg, ids, w)
    torch.cuda.synchronize()
    return to_np(ids), to_np(w)


@pytest.mark.parametrize("E,k", [(1024, 32), (1000, 31), (1024, 1), (33, 32)])
def test_softmax_select_at_limits(E, k):
    import combine_dp_gather_amd as m
    rng = np.random.default_rng(E + k)
    G = 700
    lg = rng.standard_normal((G, E)).astype(np.float32)
    lg[::5, 10:20] = lg[::5, 3:4]                      # exact ties across a block of ids
    rv = np.ones(G, np.int32)
    rv[::13] = 0
    say(f"[limits] softmax E={E} k={k}")
    ids, w = _select(m, lg, m.make_route_cfg("softmax", E, k), rv=rv)
    ref_ids, ref_w = oracle.select_softmax(lg, k, False, row_valid=rv)
    assert np.array_equal(ids, ref_ids)
    assert oracle.rel_err(w, ref_w) < 1e-6


@pytest.mark.parametrize("E,groups,topk_group,topn,k", [(1024, 64, 8, 4, 32), (1024, 64, 64, 1, 32),
                                                         (960, 60, 2, 3, 30)])
def test_grouped_select_at_limits(E, groups, topk_group, topn, k):
    import combine_dp_gather_amd as m
    rng = np.random.default_rng(E + groups + k)
    G = 500
    lg = rng.standard_normal((G, E)).astype(np.float32)
    lg[::7] = np.round(lg[::7])                        # many equal keys
    bias = (rng.uniform(-0.1, 0.1, E)).astype(np.float32)
    say(f"[limits] grouped E={E} groups={groups} topk_group={topk_group} topn={topn} k={k}")
    cfg = m.make_route_cfg("grouped", E, k, groups, topk_group, topn, True)
    ids, w = _select(m, lg, cfg, bias=bias)
    ref_ids, ref_w = oracle.select_grouped(lg, bias, groups, topk_group, k, True, group_topn=topn)
    assert np.array_equal(ids, ref_ids)
    assert oracle.rel_err(w, ref_w) < 1e-6


@pytest.mark.parametrize("replicas,mode", [(40, "sum"), (256, "max")])
def test_layer_with_1024_local_slots_and_many_replicas(replicas, mode):
    """Softmax top-8 over 1024 experts, all 1024 held as local slots, with 40 or 256 ragged
    replicas (some idle): gather and scatter run several batched launches, dispatch counts
    1024 slots, and the grouped GEMMs number 1024 segments' tiles on the device."""
    from test_gpu_parity import run_and_compare_inputs
    rng = np.random.default_rng(replicas)
    tokens = tuple(int(v) for v in rng.integers(0, 4 if replicas > 100 else 60, replicas))
    cfg = replace(moe_synth.CONFIGS["cfg2"], num_tokens=tokens, hidden=256, inter=128, num_experts=1024,
                  num_local=1024, top_k=8, name=f"limits-{replicas}r")
    run_and_compare_inputs(moe_synth.make_inputs(cfg), mode)


def test_entry_gather_many_replicas():
    """The fused entry step over 100 ragged replicas (4 launches of 32)."""
    from test_gpu_entry import _run
    rng = np.random.default_rng(100)
    tokens = tuple(int(v) for v in rng.integers(0, 30, 100))
    cfg = replace(moe_synth.CONFIGS["cfg2"], num_tokens=tokens, hidden=1024, name="entry-100r")
    _run(cfg, "max")
