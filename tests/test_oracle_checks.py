"""Pins of the parity checks themselves: the per-row relative error, the bf16 spacing, and
the element-wise bound the GPU's combine is held to.  A check that cannot see a dropped
low-weight pair would let a broken combine pass, so that case is built here on the CPU
from oracle outputs."""
import numpy as np

import moe_synth
import oracle


def test_row_rel_err_closed_forms():
    ref = np.array([[1.0, -2.0, 0.5], [0.01, 0.02, -0.01], [0.0, 0.0, 0.0]])
    assert oracle.row_rel_err(ref, ref) == 0.0
    got = ref.copy()
    got[1, 1] += 0.001                      # 5% of that row's largest value
    assert abs(oracle.row_rel_err(got, ref) - 0.05) < 1e-12
    assert oracle.rel_err(got, ref) < 1e-3  # the tensor-level figure hides it
    got = ref.copy()
    got[2, 0] = 1e-3                        # an all-zero reference row counts absolutely
    assert oracle.row_rel_err(got, ref) == 1e-3


def test_bf16_ulp_is_the_spacing_of_bf16_values():
    rng = np.random.default_rng(0)
    bits = rng.integers(0x0080, 0x7f7f, size=2000).astype(np.uint32)   # positive normal bf16
    lo = (bits << 16).view(np.float32).astype(np.float64)
    hi = ((bits + 1) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(oracle.bf16_ulp(lo), hi - lo)
    assert np.array_equal(oracle.bf16_ulp(-lo), hi - lo)
    # subnormal bf16 spacing below 2^-126
    assert oracle.bf16_ulp(np.array([0.0, 2.0 ** -130]))[0] == 2.0 ** -133


def _combine_fp32_bf16(y, w, pair_row, k):
    """The GPU's arithmetic written out: per row, an fp32 fused multiply-add chain over j
    ascending (products of fp32 weights and bf16 values are exact in float64, and one
    float64 add then one rounding to fp32 stands in for the fused step), then bf16 RNE."""
    G = len(pair_row) // k
    pr = pair_row.reshape(G, k)
    acc = np.zeros((G, y.shape[1]), dtype=np.float32)
    for j in range(k):
        m = pr[:, j] >= 0
        acc[m] = (acc[m].astype(np.float64) + w[m, j:j + 1].astype(np.float64) * y[pr[m, j]]).astype(np.float32)
    return oracle.as_f32(oracle.bf16_rne(acc.astype(np.float64)))


def _within_combine_bound(got, y, w, pair_row, k):
    ref = oracle.combine(y, {"k": k, "pair_row": pair_row}, w, len(pair_row) // k)
    mag = oracle.combine(np.abs(y), {"k": k, "pair_row": pair_row}, np.abs(w), len(pair_row) // k)
    bound = oracle.bf16_ulp(ref) + 2 * (k + 1) * 2.0 ** -24 * mag
    return np.abs(got.astype(np.float64) - ref) <= bound


def test_combine_bound_passes_gpu_arithmetic_and_catches_a_dropped_pair():
    cfg = moe_synth.CONFIGS["cfg2"]
    inp = moe_synth.make_inputs(cfg)
    res = oracle.run_layer(inp, "sum")
    plan, k = res["plan"], cfg.top_k
    # bf16 expert outputs as the GPU would hold them, the oracle's fp32 weights
    y = oracle.as_f32(oracle.bf16_rne(res["y_perm"])).astype(np.float64)
    w = res["weights"].astype(np.float32)
    pr = plan["pair_row"].copy()
    out = _combine_fp32_bf16(y, w, pr, k)
    assert np.all(_within_combine_bound(out, y, w, pr, k))
    # drop the lowest-weight local pair of the batch
    local = np.flatnonzero(pr >= 0)
    f = local[np.argmin(w.reshape(-1)[local])]
    assert w.reshape(-1)[f] < 0.03
    dropped = pr.copy()
    dropped[f] = -1
    bad = _combine_fp32_bf16(y, w, dropped, k)
    ok = _within_combine_bound(bad, y, w, pr, k)
    assert not np.all(ok[f // k])
    assert np.all(np.delete(ok, f // k, axis=0))
    # the per-row figure sees it too
    ref = oracle.combine(y, {"k": k, "pair_row": pr}, w, len(pr) // k)
    assert oracle.row_rel_err(bad, ref) > 2e-2
    print("tensor-level error of the dropped pair:", oracle.rel_err(bad, ref))
