"""GPU parity of the EPLB statistics, and one placement cycle driving the skewed fp8
workload's slot map.

Counts are integers: bit-exact against the oracle.  The placement is host code and is
checked against the oracle on the CPU; here it runs on counts the GPU produced, and must
equal the oracle's placement on the oracle's counts.  The layer step under the new map is
then held to the usual parity bar."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import moe_synth
import oracle
from gpu_helpers import build_layer, replicas_to_device, say, to_np

pytestmark = pytest.mark.gpu

# placement of the skewed workload: 256 experts in 8 groups on 288 slots (32 redundant),
# 2 nodes x 9 GPUs of 16 slots; this GPU is GPU 0, slots [0, 16)
P, GROUPS, NODES, GPUS = 288, 8, 2, 18


def _map_tensors(phys_of, n_rep):
    return torch.from_numpy(np.ascontiguousarray(phys_of)).cuda(), torch.from_numpy(np.ascontiguousarray(n_rep)).cuda()


@pytest.mark.parametrize("case", ["trivial", "replicated", "wide"])
def test_expert_load_counts(case):
    import combine_dp_gather_amd as m
    rng = np.random.default_rng(7)
    if case == "trivial":
        E, G, k, Pn, mr = 256, 5000, 8, 256, 1
        phys_of = np.arange(E, dtype=np.int32)[:, None]
        n_rep = np.ones(E, np.int32)
    elif case == "replicated":
        E, G, k, Pn, mr = 64, 3001, 6, 100, 3
        n_rep = rng.integers(1, 4, E).astype(np.int32)
        phys_of = np.full((E, 3), -1, np.int32)
        for e in range(E):
            phys_of[e, :n_rep[e]] = rng.choice(Pn + 4, n_rep[e], replace=False)  # a few slots out of range
    else:
        E, G, k, Pn, mr = 1024, 20000, 8, 8192, 8
        n_rep = rng.integers(1, 9, E).astype(np.int32)
        phys_of = np.full((E, 8), -1, np.int32)
        for e in range(E):
            phys_of[e, :n_rep[e]] = rng.choice(Pn, n_rep[e], replace=False)
    say(f"[eplb] counts {case}: E={E} G={G} k={k} P={Pn}")
    ids = rng.integers(-1, E, (G, k)).astype(np.int32)
    ids[::7] = -1                                                    # pad rows
    po, nr = _map_tensors(phys_of, n_rep)
    emap = m.make_expert_map(E, 0, 1, po, nr)
    counts = torch.zeros(Pn, dtype=torch.int64, device="cuda")
    ids_d = torch.from_numpy(ids).cuda()
    m.moe_expert_load(ids_d, emap, Pn, counts)
    torch.cuda.synchronize()
    want = oracle.physical_counts(ids, phys_of, n_rep, Pn)
    assert np.array_equal(to_np(counts), want)
    m.moe_expert_load(ids_d, emap, Pn, counts)                       # accumulates
    torch.cuda.synchronize()
    assert np.array_equal(to_np(counts), 2 * want)


def test_physical_to_logical_count():
    import combine_dp_gather_amd as m
    rng = np.random.default_rng(3)
    L, Pn, E = 5, 288, 256
    phy2log = rng.integers(0, E, (L, Pn)).astype(np.int32)
    phy2log[1, :3] = [-1, E, 9999]                                   # skipped entries
    pc = rng.integers(0, 1 << 40, (L, Pn)).astype(np.int64)
    out = torch.full((L, E), -5, dtype=torch.int64, device="cuda")
    m.moe_physical_to_logical_count(torch.from_numpy(pc).cuda(), torch.from_numpy(phy2log).cuda(), out)
    torch.cuda.synchronize()
    ok = (phy2log >= 0) & (phy2log < E)
    want = np.stack([oracle.physical_to_logical_count(np.where(ok[l], pc[l], 0)[None], np.where(ok[l], phy2log[l], 0)[None], E)[0]
                     for l in range(L)])
    assert np.array_equal(to_np(out), want)


def _hand_placement(cfg):
    """phy2log of the workload's own slot table (slots 0..15 as listed, every other expert one
    slot after them): the placement the statistics window runs under."""
    phys_of, n_rep = moe_synth.expert_map(cfg)
    Ph = int(phys_of.max()) + 1
    phy2log = np.empty(Ph, np.int32)
    for e in range(cfg.num_experts):
        for r in range(n_rep[e]):
            phy2log[phys_of[e, r]] = e
    return phys_of, n_rep, Ph, phy2log


def test_eplb_cycle_drives_the_skewed_workload():
    """Count one step of the skewed workload on the GPU under its own slot table, turn the
    counts into logical loads on the GPU, place the experts with the library, and run the
    step again under the new table: counts, loads and placement equal the oracle's, the
    balancedness over 18 GPUs improves, and the new step meets the parity bar."""
    import combine_dp_gather_amd as m
    cfg = replace(moe_synth.CONFIGS["cfg5"], num_tokens=(512,) * 8, name="skewed-fp8-eplb")
    inp = moe_synth.make_inputs(cfg)
    layer = build_layer(inp, "sum")
    layer.forward(replicas_to_device(inp))
    torch.cuda.synchronize()
    E, G, k = cfg.num_experts, layer.G, cfg.top_k
    ids = to_np(layer.topk_ids)[:G]
    phys_h, nrep_h, Ph, p2l_h = _hand_placement(cfg)
    # statistics window: one step
    counts = torch.zeros(Ph, dtype=torch.int64, device="cuda")
    m.moe_expert_load(layer.topk_ids[:G], layer.emap, Ph, counts)
    logical = torch.empty((1, E), dtype=torch.int64, device="cuda")
    m.moe_physical_to_logical_count(counts[None], torch.from_numpy(p2l_h[None]).cuda(), logical)
    torch.cuda.synchronize()
    pc_o = oracle.physical_counts(ids, phys_h, nrep_h, Ph)
    lc_o = oracle.physical_to_logical_count(pc_o[None], p2l_h[None], E)
    assert np.array_equal(to_np(counts), pc_o) and np.array_equal(to_np(logical), lc_o)
    # placement
    p2l, rank, cnt = m.moe_eplb_rebalance(to_np(logical).astype(np.float64), P, GROUPS, NODES, GPUS)
    p2l_o, rank_o, cnt_o = oracle.rebalance_hierarchical(lc_o.astype(np.float64), P, GROUPS, NODES, GPUS)
    assert np.array_equal(p2l, p2l_o) and np.array_equal(rank, rank_o) and np.array_equal(cnt, cnt_o)
    mr = int(cnt.max())
    phys_of, n_rep = m.moe_eplb_logical_to_physical(p2l[0], rank[0], E, mr)
    # balancedness over the 18 GPUs: the old table (its 260 slots padded to 288) vs the new one
    before = oracle.utilization_rate(oracle.gpu_counts(np.concatenate([pc_o, np.zeros(P - Ph, np.int64)]), GPUS))
    pc_new = oracle.physical_counts(ids, phys_of, n_rep, P)
    after = m.moe_eplb_balancedness(pc_new[None], GPUS)[0]
    assert after == oracle.utilization_rate(oracle.gpu_counts(pc_new, GPUS))
    say(f"  balancedness over {GPUS} GPUs: {before:.3f} -> {after:.3f}; this GPU's slots hold {p2l[0, :16].tolist()}")
    assert after > before
    # the step under the new table: slot s of this GPU holds logical p2l[0, s]
    cfg2 = replace(cfg, slot_logical=tuple(int(v) for v in p2l[0, :cfg.num_local]))
    inp2 = moe_synth.make_inputs(cfg2)
    inp2.phys_of, inp2.n_rep = phys_of, n_rep
    from test_gpu_parity import run_and_compare_inputs
    run_and_compare_inputs(inp2, "sum")
