"""Pins of the oracle's fused entry step (residual add + RMSNorm + DP gather) and of its
bf16 rounding, against exact rational arithmetic, closed forms and invariants."""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _bf16_value(bits):
    return float(oracle.as_f32(np.array([bits], dtype=np.uint16))[0])


# ------------------------------------------------------------------ bf16 rounding

def test_bf16_rne_round_trips_every_normal_value():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    keep = (exp != 0) & (exp != 0xFF)  # normal numbers (zero, subnormals, inf, nan excluded)
    vals = oracle.as_f32(bits[keep]).astype(np.float64)
    assert np.array_equal(oracle.bf16_rne(vals), bits[keep])
    assert oracle.bf16_rne(np.array([0.0]))[0] == 0
    assert oracle.bf16_rne(np.array([-0.0]))[0] == 0x8000


def test_bf16_rne_ties_go_to_even():
    rng = np.random.default_rng(3)
    for b in rng.integers(0x0080, 0x7F00, 500):
        b = int(b)
        lo, hi = _bf16_value(b), _bf16_value(b + 1)  # consecutive positive values
        mid = (Fraction(lo) + Fraction(hi)) / 2      # exact in float64
        got = int(oracle.bf16_rne(np.array([float(mid)]))[0])
        assert got == (b if b % 2 == 0 else b + 1)
        got_neg = int(oracle.bf16_rne(np.array([-float(mid)]))[0])
        assert got_neg == got | 0x8000


def test_bf16_rne_is_nearest_exactly():
    """Against exact rational distances to both bf16 neighbours, on random float64 values
    with all 52 fraction bits in play."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal(3000) * np.exp2(rng.integers(-60, 60, 3000))
    got = oracle.bf16_rne(x)
    for v, g in zip(x, got):
        fv = Fraction(float(v))
        mag = abs(fv)
        e = 0
        while Fraction(2) ** (e + 1) <= mag:
            e += 1
        while Fraction(2) ** e > mag:
            e -= 1
        ulp = Fraction(2) ** (e - 7)
        down = (mag // ulp) * ulp
        up = down + ulp
        if mag - down < up - mag:
            want = down
        elif mag - down > up - mag:
            want = up
        else:
            want = down if (down / ulp) % 2 == 0 else up
        want = want if fv > 0 else -want
        assert Fraction(_bf16_value(int(g))) == want


# ------------------------------------------------------------------ the entry step

def _bf(vals):
    return oracle.bf16_rne(np.asarray(vals, dtype=np.float64))


def _one(hidden, residual, gamma, eps):
    n, H = hidden.shape
    layout = oracle.gather_layout([n], "sum")
    return oracle.entry_gather(layout, [hidden], [residual], gamma, eps, H)


def test_entry_two_spikes_closed_form():
    """hidden = a at column j, residual = b at column k: the updated residual holds exactly
    a and b, and the normalised row is gamma * v / sqrt((a^2 + b^2) / H + eps) there, 0
    elsewhere.  A norm of the pre-add value, a sum instead of a mean, eps outside the root or
    a missing weight each fail it."""
    H, eps = 256, 1e-6
    rng = np.random.default_rng(11)
    gamma = _bf(rng.uniform(0.5, 1.5, H))
    g = oracle.as_f32(gamma).astype(np.float64)
    for a, b, j, k in [(1.5, -0.25, 3, 200), (2.0 ** -9, 2.0 ** -10, 0, 255), (96.0, 0.75, 17, 18)]:
        h = np.zeros((1, H)); h[0, j] = a
        r = np.zeros((1, H)); r[0, k] = b
        x, valid, res = _one(_bf(h), _bf(r), gamma, eps)
        want_res = np.zeros((1, H)); want_res[0, j] = a; want_res[0, k] = b
        assert np.array_equal(res[0], _bf(want_res))
        den = np.sqrt((a * a + b * b) / H + eps)
        want = np.zeros(H); want[j] = g[j] * a / den; want[k] = g[k] * b / den
        assert np.allclose(x[0], want, rtol=1e-13, atol=0)
        assert valid.tolist() == [1]


def test_entry_constant_rows_and_eps_inside_the_root():
    H = 128
    gamma = _bf(np.linspace(0.5, 2.0, H))
    g = oracle.as_f32(gamma).astype(np.float64)
    for c, eps in [(3.0, 1e-6), (2.0 ** -10, 1e-6), (-0.5, 0.0)]:
        r = _bf(np.full((2, H), c))
        h = _bf(np.zeros((2, H)))
        x, _, res = _one(h, r, gamma, eps)
        assert np.array_equal(res[0], r)
        assert np.allclose(x, np.tile(g * c / np.sqrt(c * c + eps), (2, 1)), rtol=1e-13, atol=0)


def test_entry_cancelled_row_is_zero_not_nan():
    H = 64
    rng = np.random.default_rng(2)
    r = _bf(rng.standard_normal((3, H)))
    h = r ^ np.uint16(0x8000)  # exact negation
    x, _, res = _one(h, r, _bf(np.ones(H)), 1e-6)
    assert np.all(oracle.as_f32(res[0]) == 0)
    assert np.all(x == 0)


def test_entry_unit_rms_and_scale_invariance():
    """With gamma = 1 and eps = 0 every output row has mean square 1, and scaling the
    residual by a power of two (exact in bf16) leaves the output unchanged."""
    H = 512
    rng = np.random.default_rng(9)
    r = _bf(rng.standard_normal((5, H)) * 3.0)
    h = _bf(np.zeros((5, H)))
    ones = _bf(np.ones(H))
    x, _, _ = _one(h, r, ones, 0.0)
    assert np.allclose(np.mean(x * x, axis=1), 1.0, rtol=1e-13)
    r4 = _bf(oracle.as_f32(r).astype(np.float64) * 4.0)
    x4, _, _ = _one(h, r4, ones, 0.0)
    assert np.allclose(x4, x, rtol=1e-14, atol=0)


def test_entry_residual_sum_matches_ieee_single_addition():
    """fp32 storage: the updated residual is the correctly rounded float32 sum, which numpy's
    float32 addition computes."""
    rng = np.random.default_rng(6)
    h = (rng.standard_normal((4, 96)) * np.exp2(rng.integers(-20, 20, (4, 96)))).astype(np.float32)
    r = (rng.standard_normal((4, 96)) * np.exp2(rng.integers(-20, 20, (4, 96)))).astype(np.float32)
    _, _, res = _one(h, r, np.ones(96, dtype=np.float32), 1e-6)
    assert np.array_equal(res[0].view(np.uint32), (h + r).view(np.uint32))


def test_entry_bf16_sum_is_rounded_exact_sum():
    """bf16 storage: the updated residual is the exact sum rounded once (checked in rational
    arithmetic on random pairs, many of which need rounding)."""
    rng = np.random.default_rng(8)
    h = _bf(rng.standard_normal((1, 400)) * np.exp2(rng.integers(-6, 6, (1, 400))))
    r = _bf(rng.standard_normal((1, 400)))
    _, _, res = _one(h, r, _bf(np.ones(400)), 1e-6)
    hv, rv = oracle.as_f32(h).astype(np.float64)[0], oracle.as_f32(r).astype(np.float64)[0]
    for j in range(400):
        exact = Fraction(float(hv[j])) + Fraction(float(rv[j]))
        got = Fraction(_bf16_value(int(res[0][0, j])))
        # nearest: no bf16 value is strictly closer than the result
        if exact != 0:
            b = int(res[0][0, j])
            for nb in (b - 1, b + 1):
                if 0 <= nb < 1 << 16 and ((nb >> 7) & 0xFF) not in (0, 0xFF) and (nb >> 15) == (b >> 15):
                    assert abs(Fraction(_bf16_value(nb)) - exact) >= abs(got - exact)
        else:
            assert got == 0


@pytest.mark.parametrize("mode", ["sum", "max"])
def test_entry_layout_and_idle_replicas(mode):
    """Rows land at the gather layout's offsets, pad rows are 0 with row_valid 0, idle
    replicas take no input and return no residual."""
    H = 32
    n = [3, 0, 5, 1]
    layout = oracle.gather_layout(n, mode)
    rng = np.random.default_rng(1)
    hid = [None if v == 0 else _bf(rng.standard_normal((v, H))) for v in n]
    res = [None if v == 0 else _bf(rng.standard_normal((v, H))) for v in n]
    gamma = _bf(rng.uniform(0.5, 1.5, H))
    x, valid, new_res = oracle.entry_gather(layout, hid, res, gamma, 1e-6, H)
    _, G, offs, sizes = layout
    assert x.shape == (G, H)
    for i, v in enumerate(n):
        if v == 0:
            assert new_res[i] is None
            continue
        xi, _, ri = _one(hid[i], res[i], gamma, 1e-6)
        assert np.array_equal(x[offs[i]:offs[i] + v], xi)
        assert np.array_equal(new_res[i], ri[0])
        assert valid[offs[i]:offs[i] + v].tolist() == [1] * v
    pad = np.ones(G, dtype=bool)
    for i, v in enumerate(n):
        pad[offs[i]:offs[i] + v] = False
    assert np.all(x[pad] == 0) and np.all(valid[pad] == 0)
