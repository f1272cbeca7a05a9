"""The no-allocation dispatch entry point, moe_dispatch_noalloc, against moe_dispatch: the
same plan and permuted rows, bit for bit, on calls in a row through the C ABI, each smaller
than the one before it (so stale tables of an earlier call sit in the fixed scratch), on the
separate-scan and fused-scan paths and the fixed-capacity layout; and its size limit,
which is refused before anything touches a GPU."""
import ctypes
import os
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def test_noalloc_rejects_problems_beyond_its_scratch():
    import combine_dp_gather_amd as m
    from combine_dp_gather_amd import _lib
    lib = m.lib()
    emap = _lib.ExpertMap(16, 1, None, None, 0, 16)
    G = 9_000_000      # 8790 blocks of 1024 pairs x 16 slots x 2 tables of int32 > 1 MiB
    assert m.moe_dispatch_workspace_size(G, 1, 16) > (1 << 20)
    plan = _lib.Plan(1, 1, 1, 1, 1, 1, 100, G, 1, 16, 1, 0)
    assert lib.moe_dispatch_noalloc(1, 1, G, 1, 64, _lib.MOE_BF16, ctypes.byref(emap), ctypes.byref(plan),
                                    1, None) == _lib.MOE_ERR_SCRATCH_LIMIT
    assert b"scratch" in lib.moe_status_string(_lib.MOE_ERR_SCRATCH_LIMIT)
    # argument errors still come first
    bad = _lib.Plan(1, 1, 1, 1, 1, 1, 100, G, 2, 16, 1, 0)
    assert lib.moe_dispatch_noalloc(1, 1, G, 1, 64, _lib.MOE_BF16, ctypes.byref(emap), ctypes.byref(bad),
                                    1, None) == _lib.MOE_ERR_INVALID_ARG


def _ids(rng, G, k, E):
    # k distinct experts per row, some rows idle (-1)
    ids = np.argsort(rng.random((G, E)), axis=1)[:, :k].astype(np.int32)
    ids[rng.random(G) < 0.05] = -1
    return ids


@pytest.mark.gpu
def test_noalloc_dispatch_equals_dispatch():
    import combine_dp_gather_amd as m
    dev = torch.device("cuda")
    rng = np.random.default_rng(42)
    # (G, k, E, E_l, first slot, H, align, seg_stride): the first needs the separate scan
    # kernel (313 blocks x 256 slots > 65536 table entries), the others the fused scan
    cases = [(40000, 8, 256, 256, 0, 256, 1, 0), (384, 8, 256, 16, 32, 7168, 128, 0),
             (200, 6, 64, 64, 0, 2048, 1, 0), (150, 8, 256, 16, 0, 512, 1, 64)]
    for G, k, E, El, p0, H, align, stride in cases:
        print(f"[noalloc] G={G} k={k} E={E} El={El} p0={p0} H={H} align={align} stride={stride}", flush=True)
        ids = torch.from_numpy(_ids(rng, G, k, E)).to(dev)
        x = torch.from_numpy(rng.standard_normal((G, H)).astype(np.float32)).to(torch.bfloat16).to(dev)
        emap = m.make_expert_map(E, p0, El)
        pa = m.PlanBuffers(G, k, El, align, device=dev, seg_stride=stride)
        pb = m.PlanBuffers(G, k, El, align, device=dev, seg_stride=stride)
        xa = torch.zeros((max(pa.cap, 1), H), dtype=torch.bfloat16, device=dev)
        xb = torch.zeros_like(xa)
        ws = torch.empty(max(m.moe_dispatch_workspace_size(G, k, El), 16), dtype=torch.uint8, device=dev)
        m.moe_dispatch(x, ids, emap, pa, xa, ws)
        m.moe_dispatch_noalloc(x, ids, emap, pb, xb)
        torch.cuda.synchronize()
        n = int(pa.num_rows.item())
        assert n == int(pb.num_rows.item()) and n > 0
        for name in ("counts", "seg_offsets", "num_rows", "error_flag", "pair_row"):
            assert torch.equal(getattr(pa, name), getattr(pb, name)), name
        assert torch.equal(pa.sorted_pair[:n], pb.sorted_pair[:n])
        assert torch.equal(xa[:n].view(torch.int16), xb[:n].view(torch.int16))
        assert int(pa.error_flag.item()) == 0
