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


def _outputs(layer):
    return [to_np(layer.global_x).copy(), to_np(layer.logits).copy(), to_np(layer.topk_ids).copy(),
            to_np(layer.plan.sorted_pair).copy(), to_np(layer.out).copy()] + \
           [to_np(y).copy() for y in layer.replicas_out]


@pytest.mark.parametrize("name", ["cfg3", "mid"])
def test_layer_step_graph_replays_bitwise(name):
    # the decode workload (static bound 24, chunk-parallel gate with its workspace) and a
    # mid-sized ragged batch on the running-total gate
    cfg = moe_synth.CONFIGS["cfg3"] if name == "cfg3" else \
        resized("cfg4", (611, 0, 1203, 377), hidden=2048, inter=1024, num_experts=64)
    say(f"[graph] {cfg.name} tokens={cfg.num_tokens}")
    inp = moe_synth.make_inputs(cfg)
    layer = build_layer(inp, "sum")
    reps = replicas_to_device(inp)
    layer.forward(reps)
    torch.cuda.synchronize()
    eager = _outputs(layer)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward(reps)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.forward(reps)
    torch.cuda.synchronize()
    for replay in range(3):
        # eager work between replays: scribble over every output of the step
        layer.out.fill_(float("nan"))
        layer.logits.fill_(float("nan"))
        layer.topk_ids.fill_(-7)
        for y in layer.replicas_out:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(_outputs(layer), eager):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), replay
    say("  3 replays bitwise equal to the eager step")
