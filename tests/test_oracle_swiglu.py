"""Pins of the SwiGLU oracle (oracle/swiglu.py) against the float64
definitions: exp and SiLU within a few fp32 ulps of their textbook values,
the bf16 activation equal to the rounded textbook value wherever that is not
within a few fp32 ulps of a bf16 rounding boundary, the gate/up layout, and
the special values."""
import math

import numpy as np
import pytest

from oracle import swiglu as S
from oracle.gemm import round_bf16


def _ulps(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    ulp = np.abs(np.spacing(ref.astype(np.float32)).astype(np.float64))
    return np.abs(got - ref) / ulp


def test_exp_within_two_ulps():
    x = np.linspace(-87.0, 88.7, 400001).astype(np.float32)
    err = _ulps(S.exp_f32(x), np.exp(x.astype(np.float64)))
    assert err.max() <= 2.0, (err.max(), x[err.argmax()])


def test_exp_special_points():
    assert S.exp_f32(np.float32(0.0)) == np.float32(1.0)
    ln_max = math.log(float(np.finfo(np.float32).max))        # 88.7228...
    assert np.isinf(S.exp_f32(np.float32(ln_max + 0.01)))
    assert np.isfinite(S.exp_f32(np.float32(ln_max - 0.01)))
    assert np.isinf(S.exp_f32(np.float32(np.inf)))
    assert np.isnan(S.exp_f32(np.float32(np.nan)))
    # below the clamp the value stays at exp(-87), a normal number
    lo = S.exp_f32(np.float32([-87.0, -200.0, -np.inf]))
    assert np.all(lo == lo[0]) and lo[0] >= np.finfo(np.float32).tiny
    # exp(1) and exp(-1): each op is rounded, so the result is e to within an ulp
    assert _ulps(S.exp_f32(np.float32(1.0)), math.e) <= 1.0
    assert _ulps(S.exp_f32(np.float32(-1.0)), 1 / math.e) <= 1.0


def test_silu_within_three_ulps():
    g = np.linspace(-80.0, 80.0, 400001).astype(np.float32)
    gd = g.astype(np.float64)
    ref = gd / (1.0 + np.exp(-gd))
    keep = np.abs(ref) > 1e-30
    err = _ulps(S.silu_f32(g)[keep], ref[keep])
    assert err.max() <= 3.0, (err.max(), g[keep][err.argmax()])


def test_silu_special_values():
    out = S.silu_f32(np.float32([0.0, -0.0, -100.0, 100.0, np.inf, -np.inf, np.nan]))
    assert out[0] == 0 and out[1] == 0 and np.signbit(out[1])
    assert out[2] == 0 and np.signbit(out[2])          # -100 / (1 + inf)
    assert out[3] == np.float32(100.0)                  # exp(-100) is tiny next to 1
    assert np.isposinf(out[4])
    assert np.isnan(out[5]) and np.isnan(out[6])        # -inf / inf, NaN in
    # silu(x) - silu(-x) = x (the odd part of x * sigmoid(x)), within rounding
    x = np.float32([0.5, 1.0, 3.0, 7.0])
    assert np.allclose(S.silu_f32(x) - S.silu_f32(-x), x, rtol=1e-6)


def _bf16_grid(rng, shape, scale):
    return round_bf16(rng.standard_normal(shape) * scale)


def test_swiglu_matches_textbook_away_from_ties():
    rng = np.random.default_rng(11)
    M, F = 512, 384
    h = _bf16_grid(rng, (M, 2 * F), 3.0)
    got = S.swiglu_bf16(h)
    g, u = h[:, :F], h[:, F:]
    exact = g / (1.0 + np.exp(-g)) * u
    ref = round_bf16(exact)
    # near a bf16 rounding boundary the fp32 steps may round either way
    eps = 8 * 2.0 ** -24
    ambiguous = round_bf16(exact * (1 + eps)) != round_bf16(exact * (1 - eps))
    assert ambiguous.mean() < 1e-3
    bad = (got != ref) & ~ambiguous
    assert not bad.any(), np.argwhere(bad)[:3]
    # where it is ambiguous the result is still one of the two neighbours
    amb = np.flatnonzero(ambiguous)
    lo = round_bf16(exact.reshape(-1)[amb] * (1 - eps))
    hi = round_bf16(exact.reshape(-1)[amb] * (1 + eps))
    gv = got.reshape(-1)[amb]
    assert np.all((gv == lo) | (gv == hi))


def test_swiglu_layout_and_zeros():
    # gate = first half, up = second half
    h = np.array([[1.0, 2.0, 2.0, 1.0]])               # g = [1, 2], u = [2, 1]
    got = S.swiglu_bf16(h)
    want = round_bf16(np.array([[2.0 / (1 + math.exp(-1.0)), 2.0 / (1 + math.exp(-2.0))]]))
    assert np.array_equal(got, want)
    swapped = S.swiglu_bf16(h[:, [2, 3, 0, 1]])
    assert not np.array_equal(swapped, got)
    # a zero gate or a zero up row gives zeros
    rng = np.random.default_rng(3)
    x = _bf16_grid(rng, (4, 64), 2.0)
    assert not S.swiglu_bf16(np.concatenate([np.zeros_like(x), x], axis=1)).any()
    assert not S.swiglu_bf16(np.concatenate([x, np.zeros_like(x)], axis=1)).any()


@pytest.mark.parametrize("F", [1, 32, 129])
def test_swiglu_shapes(F):
    h = np.ones((3, 2 * F))
    out = S.swiglu_bf16(h)
    assert out.shape == (3, F)
    assert np.all(out == round_bf16(np.float64(np.float32(1.0) / np.float32(1 + np.float32(math.exp(-1))))))
