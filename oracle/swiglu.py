"""SwiGLU between the two expert GEMMs (test infrastructure: the reference
for the fused "SwiGLU, then quantize the down-projection input" pass and
for the plain SwiGLU kernel).

Source: the Megatron-LM MoE bug report ("Loss difference when training with
FP8 vs. BF16 MoE", reproduction steps) trains Mixtral 8x7B, whose experts
apply SwiGLU between the gate/up GEMM and the down GEMM; the pages print no
formula for it. Readings taken here:

* the gate/up GEMM output ``h`` has 2F columns: the first F are the gate
  ``g``, the last F the up projection ``u`` (the two halves of a fused
  gate/up weight), and the activation is ``silu(g) * u`` with
  ``silu(g) = g * sigmoid(g) = g / (1 + exp(-g))``;
* the activation is the bf16 value nearest to the exact real number
  ``silu(g) * u`` (ties to even), i.e. a correctly rounded bf16 result.
  For finite bf16 ``g != 0`` and ``u != 0`` that number is transcendental
  (``exp`` of a nonzero rational is), so it is never a bf16 midpoint and
  the rounding is unambiguous; ``g == 0`` or ``u == 0`` gives a signed
  zero. NaN and infinite inputs follow float64 arithmetic on the same
  formula (``g = -inf`` gives NaN, as ``-inf * 0``).

How it is computed: the formula in float64 (relative error below 2^-50),
rounded directly to bf16 (``gemm.round_bf16``, no float32 step); where that
float64 value lies within 2^-40 of its size from a bf16 rounding midpoint,
the element is recomputed with Python's ``decimal`` module at 120 digits
(its ``exp`` is correctly rounded at that precision) and rounded by exact
comparison with the midpoint. Nothing here is tuned to any device
algorithm.
"""
from __future__ import annotations

import decimal
import math

import numpy as np

from .gemm import round_bf16

TIE_REL = 2.0 ** -40       # float64 values this close to a bf16 midpoint are recomputed exactly
_PREC = 120                # decimal digits (2^-133, the bf16 subnormal quantum, has 93)


def sigmoid_f64(g) -> np.ndarray:
    """sigmoid(g) = 1 / (1 + exp(-g)) in float64, evaluated as
    exp(g) / (1 + exp(g)) for g < 0 (the same value, without overflow)."""
    g = np.asarray(g, np.float64)
    e = np.exp(-np.abs(g))
    with np.errstate(invalid="ignore"):
        return np.where(g >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def silu_f64(g) -> np.ndarray:
    """silu(g) = g * sigmoid(g) in float64."""
    g = np.asarray(g, np.float64)
    with np.errstate(invalid="ignore"):
        return g * sigmoid_f64(g)


def _bf16_quantum(a: np.ndarray) -> np.ndarray:
    """Spacing of the bf16 values around |a| (8 significant bits; a fixed
    2^-133 below the smallest normal 2^-126)."""
    e = np.frexp(a)[1] - 1                       # a in [2^e, 2^(e+1))
    return np.ldexp(1.0, np.maximum(e, -126) - 7)


def near_midpoint(p) -> np.ndarray:
    """True where the float64 value p lies within TIE_REL * |p| of a bf16
    rounding midpoint (where its own rounding error could decide the
    bf16 result)."""
    p = np.asarray(p, np.float64)
    a = np.abs(p)
    ok = np.isfinite(a) & (a > 0)
    q = _bf16_quantum(np.where(ok, a, 1.0))
    t = np.where(ok, a, 1.0) / q
    frac = t - np.floor(t)
    return ok & (np.abs(frac - 0.5) * q <= TIE_REL * np.where(ok, a, 1.0))


def swiglu_exact_bf16(g: float, u: float) -> float:
    """The bf16 value nearest to silu(g) * u for finite g, u, by exact
    decimal arithmetic (returned as a float)."""
    if g == 0 or u == 0:
        return float(np.float64(g) * 0.5 * np.float64(u))       # signed zero, as IEEE gives it
    ctx = decimal.Context(prec=_PREC)
    D = decimal.Decimal
    gd, ud = D(float(g)), D(float(u))
    if g >= 0:
        p = ctx.divide(ctx.multiply(gd, ud), ctx.add(D(1), ctx.exp(ctx.minus(gd))))
    else:
        eg = ctx.exp(gd)
        p = ctx.divide(ctx.multiply(ctx.multiply(gd, ud), eg), ctx.add(D(1), eg))
    a = ctx.copy_abs(p)                       # every step in the 120-digit context
    approx = float(a)
    q = float(_bf16_quantum(np.float64(approx)))
    k = math.floor(ctx.divide(a, D(q)))
    mid = ctx.multiply(ctx.add(D(k), D("0.5")), D(q))           # exact: q is a power of two
    if a == mid:
        # only when exp(-g) is below the working precision (g beyond ~276),
        # 1 + exp(-g) rounds to 1 and |g u| (exact) is the midpoint itself;
        # the true |silu(g) * u| = |g u| sigmoid(g) is strictly smaller, since
        # sigmoid(g) < 1, so it rounds toward zero
        assert g > 0 and ctx.copy_abs(ctx.multiply(gd, ud)) == mid, "silu(g) * u is never a bf16 midpoint"
        r = k * q
    else:
        r = (k + 1) * q if a > mid else k * q
    if abs(r) >= 2.0 ** 128:                  # past the largest bf16: rounds to infinity
        r = math.inf
    return math.copysign(r, float(p))


def swiglu_bf16(h) -> np.ndarray:
    """Activation [M, F] (bf16 values as float64) of a gate/up output h
    [M, 2F] given as float values (bf16-representable)."""
    h = np.asarray(h, np.float64)
    F = h.shape[-1] // 2
    g, u = h[..., :F], h[..., F:]
    with np.errstate(invalid="ignore", over="ignore"):
        p = silu_f64(g) * u
    out = round_bf16(p)
    amb = near_midpoint(p) & np.isfinite(g) & np.isfinite(u)
    for idx in zip(*np.nonzero(amb)):
        out[idx] = swiglu_exact_bf16(float(g[idx]), float(u[idx]))
    return out
