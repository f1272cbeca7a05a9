"""The six calls captured in one HIP graph: no call allocates, copies or synchronises the
host, so a layer step can be captured once and replayed (what a decode loop at a static
batch bound does to remove launch overhead).  Each replay is checked bit for bit against
the eager step, with eager kernels overwriting the outputs and host synchronisations
between the replays."""
import numpy as np
import pytest
import torch

import moe_synth
from gpu_helpers import build_layer, replicas_to_device, resized, say, to_np

pytestmark = pytest.mark.gpu


def _outputs(layer, with_out=True):
    # sorted_pair is defined up to num_rows; rows past it keep whatever an earlier step left
    rows = int(to_np(layer.plan.num_rows)[0])
    return [to_np(layer.global_x).copy(), to_np(layer.logits).copy(), to_np(layer.topk_ids).copy(),
            to_np(layer.plan.sorted_pair)[:rows].copy()] + \
           ([to_np(layer.out).copy()] if with_out else []) + [to_np(y).copy() for y in layer.replicas_out]


@pytest.mark.parametrize("name", ["cfg3", "mid", "cfg3-fixed", "cfg3-entry", "cfg3-exit", "cfg4"])
def test_layer_step_graph_replays_bitwise(name):
    # the decode workload (static bound 24, the 16x16-chain gate), a
    # mid-sized ragged batch, the decode workload in the
    # fixed-capacity layout (16 slots x 384 rows), the decode workload with the fused
    # entry step (its residual is restored before every run, since the step updates it), the
    # decode workload with the fused exit (the global output buffer is then not written),
    # and the whole prefill batch (8 x 4096 rows, H = 7168), the step bench.py replays
    if name == "mid":
        cfg = resized("cfg4", (611, 0, 1203, 377), hidden=2048, inter=1024, num_experts=64)
    else:
        cfg = moe_synth.CONFIGS["cfg4" if name == "cfg4" else "cfg3"]
    say(f"[graph] {name}: {cfg.name} tokens={cfg.num_tokens}")
    inp = moe_synth.make_inputs(cfg)
    layer = build_layer(inp, "sum", seg_stride=384 if name == "cfg3-fixed" else 0)
    reps = replicas_to_device(inp)
    entry, res0 = None, None
    if name == "cfg3-entry":
        ent = moe_synth.make_entry_inputs(cfg, inp.replicas)
        res0 = [torch.from_numpy(r).view(torch.bfloat16).cuda() for r in ent.residual]
        res = [r.clone() for r in res0]
        entry = (res, torch.from_numpy(ent.gamma).view(torch.bfloat16).cuda(), ent.eps)

    def restore():
        if res0 is not None:
            for a, b in zip(entry[0], res0):
                a.copy_(b)

    fused_exit = name == "cfg3-exit"

    def outputs():
        return _outputs(layer, not fused_exit) + ([to_np(r).copy() for r in entry[0]] if entry else [])

    layer.forward(reps, entry, fused_exit)
    torch.cuda.synchronize()
    eager = outputs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward(reps, entry, fused_exit)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.forward(reps, entry, fused_exit)
    torch.cuda.synchronize()
    for replay in range(3):
        # eager work between replays: scribble over every output of the step
        restore()
        layer.out.fill_(float("nan"))
        layer.logits.fill_(float("nan"))
        layer.topk_ids.fill_(-7)
        for y in layer.replicas_out:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outputs(), eager)):
            diff = int(np.count_nonzero(a.view(np.uint8) != b.view(np.uint8)))
            assert diff == 0, f"replay {replay}: output {i} differs in {diff} of {a.nbytes} bytes"
    say("  3 replays bitwise equal to the eager step")
