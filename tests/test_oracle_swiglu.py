"""Pins of the SwiGLU oracle (oracle/swiglu.py): the bf16 value nearest to
silu(g) * u, silu(g) = g / (1 + exp(-g)), for bf16 gate and up values.

What pins it, besides its own formula:
* sigmoid against scipy's ``expit`` (a library routine, computed without
  the oracle's exp(-|g|) split);
* values worked by hand from e = 2.718281828459045... and the bf16 grid;
* the exact (decimal) evaluation and the float64 evaluation agree wherever
  the float64 value is not near a bf16 midpoint, and the decimal one obeys
  silu(x) - silu(-x) = x;
* products g * u that are exact bf16 midpoints with g large: the true value
  lies just below |g * u| (sigmoid(g) < 1), so it must round toward zero,
  where float64 alone (1 + exp(-g) == 1) would see an exact tie and round
  to even, away from zero;
* signed zeros, underflow, overflow and the gate/up layout."""
import math

import numpy as np
import pytest

from oracle import swiglu as S
from oracle.gemm import round_bf16

scipy_special = pytest.importorskip("scipy.special")


def _bf16_values(bits):
    with np.errstate(invalid="ignore"):
        return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


ALL_BF16 = _bf16_values(np.arange(65536, dtype=np.uint32).astype(np.uint16))
FINITE_BF16 = ALL_BF16[np.isfinite(ALL_BF16)]


def test_sigmoid_matches_expit_on_every_bf16_gate():
    g = FINITE_BF16[np.abs(FINITE_BF16) <= 700]
    ref = scipy_special.expit(g)
    got = S.sigmoid_f64(g)
    keep = ref > 1e-300
    rel = np.abs(got[keep] - ref[keep]) / ref[keep]
    assert rel.max() <= 4e-16, (rel.max(), g[keep][rel.argmax()])


def test_hand_worked_points():
    """silu(g) * u for small arguments, rounded on the bf16 grid by hand.
    With e = 2.718281828459045:
      sigmoid(1)  = 1 / (1 + 1/e) = 0.7310585786300049; bf16 spacing in
        [0.5, 1) is 2^-8, 0.73105858 / 2^-8 = 187.15 -> 187 * 2^-8 = 0.73046875;
      silu(-1)    = -1 / (1 + e)  = -0.2689414213699951; spacing in
        [0.25, 0.5) is 2^-9, 137.70 -> 138 * 2^-9 = 0.26953125 (negative);
      silu(2) * 3 = 6 / (1 + e^-2) = 5.284782467867294; spacing in [4, 8)
        is 2^-5, 169.11 -> 169 * 2^-5 = 5.28125;
      silu(-4) * -2 = 8 e^-4 / (1 + e^-4) = 0.14388...; e^-4 = 0.01831563888873418,
        8 * 0.018315639 / 1.018315639 = 0.14388800...; spacing in [0.125, 0.25)
        is 2^-10, 147.34 -> 147 * 2^-10 = 0.1435546875;
      silu(0.5) * 1 = 0.5 / (1 + e^-0.5) = 0.5 / 1.6065306597126334 =
        0.31122966560092726; spacing 2^-9, 159.35 -> 159 * 2^-9 = 0.310546875."""
    h = np.array([[1.0, -1.0, 2.0, -4.0, 0.5, 1.0, 1.0, 3.0, -2.0, 1.0]])
    got = S.swiglu_bf16(h)[0]
    want = [0.73046875, -0.26953125, 5.28125, 0.1435546875, 0.310546875]
    assert got.tolist() == want
    for (g, u), w in zip([(1.0, 1.0), (-1.0, 1.0), (2.0, 3.0), (-4.0, -2.0), (0.5, 1.0)], want):
        assert S.swiglu_exact_bf16(g, u) == w


def _false_ties(sign_g=1):
    """bf16 pairs (g, u), g >= 40, with g * u an exact bf16 midpoint whose
    ties-to-even neighbour is the one away from zero."""
    out = []
    gs = _bf16_values(np.arange(0x4220, 0x4300, 7, dtype=np.uint32).astype(np.uint16))   # 40 .. 128
    us = _bf16_values(np.arange(0x3F80, 0x4000, dtype=np.uint32).astype(np.uint16))      # 1 .. 2
    for g in gs:
        for u in us:
            p = g * u                                    # exact: 8 x 8 significant bits
            q = float(S._bf16_quantum(np.float64(p)))
            k, r = divmod(p, q)
            if r == q / 2 and int(k) % 2 == 1:           # midpoint; even neighbour is k + 1 (away)
                out.append((sign_g * g, u, k * q))
    return out


def test_midpoint_products_round_toward_zero():
    cases = _false_ties()
    assert len(cases) > 20
    for g, u, toward_zero in cases[:200]:
        for sg, su in ((1, 1), (1, -1)):
            gg, uu = sg * g, su * u
            want = math.copysign(toward_zero, gg * uu)
            assert S.swiglu_exact_bf16(gg, uu) == want, (gg, uu)
            assert S.swiglu_bf16(np.array([[gg, uu]]))[0, 0] == want, (gg, uu)
            # float64 alone sees an exact tie (1 + exp(-g) == 1) and rounds away from zero
            p64 = S.silu_f64(np.float64(gg)) * uu
            assert p64 == gg * uu and round_bf16(np.float64(p64)) != want


def test_midpoint_products_beyond_the_decimal_exponent_range():
    """g = 1.5 * 2^100: exp(-g) underflows even in decimal arithmetic; g * u
    with u = 1 + 2^-7 is the midpoint (1 + 65.5/128) 2^100, and sigmoid(g) < 1
    puts the value below it: (1 + 65/128) 2^100 (ties-to-even would give 66)."""
    g, u = 1.5 * 2.0 ** 100, 1 + 2.0 ** -7
    want = (1 + 65 / 128) * 2.0 ** 100
    assert S.swiglu_exact_bf16(g, u) == want and S.swiglu_exact_bf16(g, -u) == -want
    assert S.swiglu_bf16(np.array([[g, u]]))[0, 0] == want
    assert round_bf16(np.float64(g * u)) == (1 + 66 / 128) * 2.0 ** 100
    # the same far beyond the bf16 range: the result is infinite, not a large finite value
    big = 1.5 * 2.0 ** 126
    assert S.swiglu_exact_bf16(big, 3.0) == np.inf and S.swiglu_exact_bf16(big, -3.0) == -np.inf
    assert S.swiglu_bf16(np.array([[big, 2.0 ** 126]]))[0, 0] == np.inf


def test_decimal_and_float64_agree_away_from_midpoints():
    rng = np.random.default_rng(5)
    n = 3000
    g = round_bf16(np.concatenate([rng.standard_normal(n) * 3.0,
                                   rng.uniform(-110, 110, n // 3),
                                   [0.0, -0.0, 1e-30, -1e-30, 88.0, -88.0, -100.0, 700.0]]))
    u = round_bf16(np.concatenate([rng.standard_normal(n) * 10.0 ** rng.integers(-30, 30, n),
                                   rng.standard_normal(n // 3) * 1e30,
                                   [1.0, 1.0, 1e30, -1e30, 1e-20, 3e38, 1e38, 2.0]]))
    with np.errstate(over="ignore", invalid="ignore"):
        p = S.silu_f64(g) * u
    near = S.near_midpoint(p)
    # float64 sees exact midpoints where g > 37 (1 + exp(-g) == 1) and g * u has
    # 9 significant bits; elsewhere a float64 value is near one with odds ~2^-31
    assert near.mean() < 1e-2
    vec = round_bf16(p)
    for gi, ui, vi, ni in zip(g, u, vec, near):
        if ni:
            continue
        assert S.swiglu_exact_bf16(gi, ui) == vi or (np.isnan(vi)), (gi, ui, vi)


def test_odd_part_identity():
    """silu(x) - silu(-x) = x (x sigmoid(x) + x sigmoid(-x), sigmoid(x) + sigmoid(-x) = 1)."""
    x = FINITE_BF16[(np.abs(FINITE_BF16) > 1e-30) & (np.abs(FINITE_BF16) < 1e30)]
    d = S.silu_f64(x) - S.silu_f64(-x)
    assert np.max(np.abs(d - x) / np.abs(x)) <= 4 * 2.0 ** -52
    import decimal
    ctx = decimal.Context(prec=60)
    for v in (0.5, 1.0, 3.25, 17.0, 41.5):
        xv = decimal.Decimal(v)
        a = ctx.divide(xv, ctx.add(1, ctx.exp(-xv)))
        b = ctx.divide(-xv, ctx.add(1, ctx.exp(xv)))
        assert abs(ctx.subtract(ctx.subtract(a, b), xv)) < decimal.Decimal("1e-55")


def test_special_values():
    h = np.array([[0.0, -0.0, 1.0, -1.0, -200.0, 2.0, np.nan, np.inf, -np.inf, 3.0,
                   1.0, 1.0, -0.0, 0.0, 3e38, 3e38, 1.0, 1.0, 1.0, 0.0]])
    out = S.swiglu_bf16(h)[0]
    assert out[0] == 0 and not np.signbit(out[0])              # +0 * 1
    assert out[1] == 0 and np.signbit(out[1])                  # -0 * 1
    assert out[2] == 0 and np.signbit(out[2])                  # silu(1) * -0
    assert out[3] == 0 and np.signbit(out[3])                  # silu(-1) * 0 = -0
    assert out[4] == 0 and np.signbit(out[4])                  # -200 e^-200 * 3e38 underflows to -0
    assert np.isposinf(out[5])                                 # silu(2) * 3e38 overflows
    assert np.isnan(out[6])                                    # NaN gate
    assert np.isposinf(out[7])                                 # silu(inf) * 1
    assert np.isnan(out[8])                                    # silu(-inf) = -inf * 0
    assert out[9] == 0                                         # silu(3) * 0


def test_layout_and_zeros():
    h = np.array([[1.0, 2.0, 2.0, 1.0]])                       # g = [1, 2], u = [2, 1]
    got = S.swiglu_bf16(h)
    want = round_bf16(np.array([[2.0 / (1 + math.exp(-1.0)), 2.0 / (1 + math.exp(-2.0))]]))
    assert np.array_equal(got, want)
    assert not np.array_equal(S.swiglu_bf16(h[:, [2, 3, 0, 1]]), got)
    rng = np.random.default_rng(3)
    x = round_bf16(rng.standard_normal((4, 64)) * 2.0)
    assert not S.swiglu_bf16(np.concatenate([np.zeros_like(x), x], axis=1)).any()
    assert not S.swiglu_bf16(np.concatenate([x, np.zeros_like(x)], axis=1)).any()


@pytest.mark.parametrize("F", [1, 32, 129])
def test_shapes(F):
    out = S.swiglu_bf16(np.ones((3, 2 * F)))
    assert out.shape == (3, F)
    assert np.all(out == 0.73046875)
