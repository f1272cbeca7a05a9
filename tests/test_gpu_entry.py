"""GPU parity of the fused entry step (residual add + RMSNorm + DP gather) against the oracle,
through the C ABI.

Bar, derived from the arithmetic:
  * the updated residual is bit-exact (one fp32 add of two stored values, then one rounding:
    the fp32 sum of two bf16 values is exact, so both sides round the exact sum);
  * row_valid and every pad row are bit-exact;
  * each normalised element is within 2^-8 + 5e-5 of the float64 value, relative (bf16):
    rounding to bf16 costs at most 2^-8 relative, and the fp32 mean of squares, root and
    products stay far below 5e-5 for rows up to 16k wide; fp32 storage: 5e-5 relative.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import moe_synth
import oracle
from gpu_helpers import act_dtype, build_layer, copy_path_rows, say, to_np

pytestmark = pytest.mark.gpu

REL_BF16 = 2.0 ** -8 + 5e-5
REL_F32 = 5e-5


def _dev(a, bf):
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t.view(torch.bfloat16) if bf else t).cuda()


def _inputs(cfg):
    inp = moe_synth.make_inputs(cfg, with_experts=False)
    ent = moe_synth.make_entry_inputs(cfg, inp.replicas)
    return inp, ent


def _check(layout, ent, H, gx, valid, res_dev, bf):
    gx_ref, valid_ref, res_ref = oracle.entry_gather(layout, ent.hidden, ent.residual, ent.gamma, ent.eps, H)
    G = layout[1]
    assert np.array_equal(to_np(valid)[:G], valid_ref)
    for i, r in enumerate(res_ref):
        if r is not None:
            got = to_np(res_dev[i])[:layout[3][i]]
            assert np.array_equal(got.view(np.uint16 if bf else np.uint32), r.view(np.uint16 if bf else np.uint32)), i
    got = oracle.as_f32(to_np(gx)).astype(np.float64)
    diff = np.abs(got - gx_ref)
    bound = (REL_BF16 if bf else REL_F32) * np.abs(gx_ref)
    worst = float(np.max(diff - bound)) if diff.size else 0.0
    say(f"  global_x: max |diff| - bound = {worst:.3e}, rel err {oracle.rel_err(got, gx_ref):.3e}")
    assert np.all(diff <= bound)
    return gx_ref


def _run(cfg, mode, alias=False, misalign=False):
    bf = cfg.dtype == "bf16"
    inp, ent = _inputs(cfg)
    H = cfg.hidden
    if alias:  # the residual buffer is also the attention output: the update doubles it
        ent = replace(ent, hidden=[r.copy() for r in ent.residual])
    import combine_dp_gather_amd as m
    L = m.moe_gather_layout(cfg.num_tokens, mode, static_bound=cfg.static_bound)
    layout = oracle.gather_layout(cfg.num_tokens, mode, static_bound=cfg.static_bound)
    G = layout[1]
    say(f"[entry] {cfg.name} tokens={cfg.num_tokens} H={H} dtype={cfg.dtype} mode={mode} G={G} "
        f"alias={alias} misalign={misalign}")
    hid = [_dev(h, bf) for h in ent.hidden]
    if misalign:
        # residual rows start 1 element past a 16-byte boundary: the two-pass path
        res = []
        for r in ent.residual:
            t = torch.empty(r.size + 1, dtype=act_dtype(cfg), device="cuda")
            v = t[1:].view(r.shape)
            v.copy_(_dev(r, bf))
            res.append(v)
    else:
        res = [_dev(r, bf) for r in ent.residual]
    if alias:
        hid = res
    gamma = _dev(ent.gamma, bf)
    gx = torch.full((max(G, 1), H), 7.0, dtype=act_dtype(cfg), device="cuda")[:G]
    valid = torch.full((max(G, 1),), 9, dtype=torch.int32, device="cuda")
    m.moe_entry_gather(L, hid, res, gamma, ent.eps, gx, valid)
    torch.cuda.synchronize()
    if G == 0:
        return
    _check(layout, ent, H, gx, valid, res, bf)


@pytest.mark.parametrize("name,mode", [("cfg1", "sum"), ("cfg2", "sum"), ("cfg2", "max"), ("cfg3", "sum")])
def test_entry_configs(name, mode):
    _run(moe_synth.CONFIGS[name], mode)


@pytest.mark.parametrize("H", [2048, 4096, 7168, 8192, 8200, 100, 8])
def test_entry_widths(H):
    """Register path at 4, 8, 14 of 16 and 16 chunks per lane (H = 2048, 4096, 7168, 8192),
    and the two-pass path for a row too wide for registers (8200) or not a multiple of 16
    bytes (100); H = 8 is one chunk, most lanes idle."""
    cfg = replace(moe_synth.CONFIGS["cfg2"], hidden=H, name=f"entry-H{H}")
    _run(cfg, "max")


def test_entry_f32_wide():
    cfg = replace(moe_synth.CONFIGS["cfg1"], hidden=7168, num_tokens=(5, 0, 9), name="entry-f32-7168")
    _run(cfg, "sum")


def test_entry_misaligned_residual_takes_two_pass_path():
    _run(moe_synth.CONFIGS["cfg2"], "sum", misalign=True)


def test_entry_residual_aliases_input():
    _run(moe_synth.CONFIGS["cfg2"], "sum", alias=True)


def test_entry_all_idle_is_noop():
    cfg = replace(moe_synth.CONFIGS["cfg2"], num_tokens=(0, 0, 0), name="entry-idle")
    _run(cfg, "sum")


def test_entry_prefill_fullsize():
    """8 replicas x 4096 tokens, H = 7168, in the launch configuration the step uses: every
    residual element bit for bit and every normalised element to the bound, one replica at a
    time on the oracle side."""
    cfg = moe_synth.CONFIGS["cfg4"]
    bf = True
    inp, ent = _inputs(cfg)
    import combine_dp_gather_amd as m
    L = m.moe_gather_layout(cfg.num_tokens, "sum")
    layout = oracle.gather_layout(cfg.num_tokens, "sum")
    say(f"[entry] full size {cfg.num_tokens} H={cfg.hidden}")
    hid = [_dev(h, bf) for h in ent.hidden]
    res = [_dev(r, bf) for r in ent.residual]
    gamma = _dev(ent.gamma, bf)
    G = layout[1]
    gx = torch.empty((G, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    valid = torch.empty(G, dtype=torch.int32, device="cuda")
    m.moe_entry_gather(L, hid, res, gamma, ent.eps, gx, valid)
    torch.cuda.synchronize()
    assert int(valid.sum().item()) == G
    offs = layout[2]
    for i, n in enumerate(cfg.num_tokens):
        one = oracle.gather_layout([n], "sum")
        sub = replace(ent, hidden=[ent.hidden[i]], residual=[ent.residual[i]])
        _check(one, sub, cfg.hidden, gx[offs[i]:offs[i] + n], valid[offs[i]:offs[i] + n], [res[i]], bf)


def test_layer_step_with_entry():
    """The whole step with the fused entry in place of the gather: the global buffer the
    later steps read is the entry step's output, and routing, dispatch, experts, combine and
    scatter then match the oracle run on exactly those rows."""
    cfg = moe_synth.CONFIGS["cfg2"]
    inp, ent = _inputs(cfg)
    full = moe_synth.make_inputs(cfg)
    layer = build_layer(full, "sum")
    bf = True
    hid = [_dev(h, bf) for h in ent.hidden]
    res = [_dev(r, bf) for r in ent.residual]
    gamma = _dev(ent.gamma, bf)
    layer.forward(hid, entry=(res, gamma, ent.eps))
    torch.cuda.synchronize()
    layout = oracle.gather_layout(cfg.num_tokens, "sum")
    _check(layout, ent, cfg.hidden, layer.global_x, layer.row_valid, res, bf)
    # the oracle's path from the GPU's normalised rows on
    gx = to_np(layer.global_x)
    offs = layout[2]
    reps = [gx[offs[i]:offs[i] + n].copy() for i, n in enumerate(cfg.num_tokens)]
    ref = oracle.run_layer(replace(full, replicas=reps), "sum")
    assert np.array_equal(to_np(layer.topk_ids)[:layer.G], ref["ids"])
    assert np.array_equal(to_np(copy_path_rows(layer)[0])[:ref["plan"]["num_rows"]], ref["x_perm"])
    out = oracle.as_f32(to_np(layer.out))
    err = oracle.rel_err(out, ref["out"])
    say(f"  out rel err {err:.3e}")
    assert err < 2e-2
