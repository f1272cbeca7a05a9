"""Shared set-up of the GPU tests: seeded inputs on the device, the layer's six calls, and
conversions of device results back to numpy for comparison with the oracle."""
from __future__ import annotations

import sys
from dataclasses import replace

import numpy as np
import torch

import moe_synth

TOL_BF16 = 2e-2     # max relative error (infinity norm) for bf16 outputs, fp32 accumulate
TOL_FP8 = 5e-2      # fp8 weights
TOL_F32 = 1e-4      # fp32 path (the oracle accumulates in fp64)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def tol_for(cfg):
    if cfg.weight_format == "fp8_block":
        return TOL_FP8
    return TOL_F32 if cfg.dtype == "f32" else TOL_BF16


def act_dtype(cfg):
    return torch.float32 if cfg.dtype == "f32" else torch.bfloat16


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.uint16).numpy()
    return t.numpy()


def replicas_to_device(inp, device="cuda"):
    bf = inp.cfg.dtype == "bf16"
    out = []
    for r in inp.replicas:
        t = torch.from_numpy(np.ascontiguousarray(r))
        if bf:
            t = t.view(torch.bfloat16)
        out.append(t.to(device))
    return out


def resized(name, tokens, **kw):
    cfg = moe_synth.CONFIGS[name]
    return replace(cfg, num_tokens=tuple(tokens), static_bound=0, name=f"{name}-{len(tokens)}r", **kw)


def build_layer(inp, mode="sum", align=1, cap=None, fp8_act="bf16", seg_stride=0, fuse_permute=True):
    from combine_dp_gather_amd.layer import DeviceWeights, MoELayer, spec_of
    cfg = inp.cfg
    w = DeviceWeights(inp, fp8_act=fp8_act)
    layer = MoELayer(spec_of(cfg), w, cfg.num_tokens, act_dtype(cfg), mode=mode,
                     static_bound=cfg.static_bound, align=align, cap=cap, seg_stride=seg_stride,
                     fuse_permute=fuse_permute)
    return layer


def copy_path_rows(layer):
    """For a layer run with the permute folded into the up GEMM: the permuted copy (moe_dispatch
    with an x_perm buffer, re-deriving the same plan from the same ids) and the plain up GEMM
    on it.  Returns (x_perm, h) of the copy path, device tensors."""
    import combine_dp_gather_amd as m
    s = layer.spec
    xp = torch.empty((max(layer.plan.cap, 1), s.hidden), dtype=layer.dt, device=layer.device)
    h = torch.empty_like(layer.h)
    m.moe_dispatch(layer.global_x, layer.topk_ids[:layer.G], layer.emap, layer.plan, xp,
                   layer.dispatch_ws)
    m.moe_expert_gemm_up(xp, layer.plan, layer.w.ew, s.hidden, s.inter, h, layer.gemm_ws)
    torch.cuda.synchronize()
    return xp, h


def check_combine_bound(out_dev, y_dev, w_dev, pair_row, k, scale=1.0, chunk=2048):
    """The device's out against the float64 combine of the device's own y_perm and weights,
    element by element: |out - ref| <= (one bf16 ulp of ref, for bf16 outputs) +
    2 (k + 1) 2^-24 |scale| sum_j |w_j y_j| -- the rounding of the output plus the fp32
    fused multiply-add chain over at most k terms and the scale.  Device arrays come as
    numpy (bf16 as uint16 bits).  Returns the largest deviation as a fraction of its bound."""
    import oracle
    G = len(pair_row) // k
    bf = out_dev.dtype == np.uint16
    y = oracle.as_f32(y_dev).astype(np.float64)
    w = np.asarray(w_dev, dtype=np.float64)
    worst = 0.0
    for g0 in range(0, G, chunk):
        g1 = min(G, g0 + chunk)
        pr = {"k": k, "pair_row": pair_row[g0 * k:g1 * k]}
        ref = oracle.combine(y, pr, w[g0:g1], g1 - g0, scale)
        mag = oracle.combine(np.abs(y), pr, np.abs(w[g0:g1]), g1 - g0, abs(scale))
        bound = 2 * (k + 1) * 2.0 ** -24 * mag + (oracle.bf16_ulp(ref) if bf else 2.0 ** -149)
        dev = np.abs(oracle.as_f32(out_dev[g0:g1]).astype(np.float64) - ref)
        assert np.all(dev <= bound), f"rows {g0}..{g1}: {int(np.sum(dev > bound))} elements past the bound"
        worst = max(worst, float(np.max(dev / bound)))
    return worst

