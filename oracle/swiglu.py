"""SwiGLU between the two expert GEMMs, in reproducible fp32 (test
infrastructure: the reference for the fused "SwiGLU, then quantize the
down-projection input" pass).

Source: the Megatron-LM MoE bug report trains Mixtral 8x7B, whose experts
apply SwiGLU between the gate/up GEMM and the down GEMM (its reproduction
steps); the pages print no formula for it. Readings taken here:

* the gate/up GEMM output ``h`` has 2F columns: the first F are the gate
  ``g``, the last F the up projection ``u`` (the split of a fused gate/up
  weight into two halves), and the activation is ``silu(g) * u`` with
  ``silu(g) = g / (1 + exp(-g))``;
* the activation is produced in bf16 (the dtype of the tensors between the
  GEMMs), rounded to nearest even from the fp32 product, and quantized from
  those bf16 values like any other activation;
* so that a device implementation can match every bit, the fp32 value is
  defined by correctly rounded fp32 operations only, in this order (no
  fused multiply-adds): an exponential by Cody-Waite range reduction with a
  two-part ln 2 and a degree-7 Taylor polynomial in Horner form, scaled by
  an exact power of two; then one add and one IEEE division for SiLU, and
  one multiply by ``u``. The exponential's argument is clamped to
  [-87, 89] first: below, the true result would be subnormal (SiLU's
  ``1 + exp(-g)`` is then 1 in fp32 anyway); above, it overflows to +inf as
  the true one does. NaN stays NaN, and ``g = -inf`` gives NaN (IEEE
  ``-inf / inf``).

numpy float32 arithmetic is IEEE single with round-to-nearest-even, so each
step below is the correctly rounded operation it names. The tests pin the
exponential and SiLU to their float64 definitions within a few fp32 ulps,
and the bf16 activation to the float64 textbook value away from bf16
rounding boundaries.
"""
from __future__ import annotations

import numpy as np

from .gemm import round_bf16

_F = np.float32

LOG2E = _F(1.4426950408889634)                    # fp32 nearest of log2(e)
LN2_HI = _F(0.693145751953125)                    # 16 significant bits: n * LN2_HI exact for |n| <= 256
LN2_LO = _F(0.6931471805599453 - 0.693145751953125)
# 1/7!, 1/6!, ..., 1/1!, 1/0! as fp32, highest degree first
TAYLOR = [_F(1.0 / 5040), _F(1.0 / 720), _F(1.0 / 120), _F(1.0 / 24), _F(1.0 / 6), _F(0.5), _F(1.0), _F(1.0)]
EXP_LO, EXP_HI = _F(-87.0), _F(89.0)


def exp_f32(x) -> np.ndarray:
    """fp32 exp(x) by the operation sequence stated in the module docstring."""
    x = np.asarray(x, np.float32)
    nan = np.isnan(x)
    xc = np.clip(np.where(nan, _F(0), x), EXP_LO, EXP_HI).astype(np.float32)
    n = np.rint(xc * LOG2E).astype(np.float32)             # nearest integer, ties to even
    r = ((xc - n * LN2_HI) - n * LN2_LO).astype(np.float32)
    p = TAYLOR[0] * np.ones_like(r)
    for c in TAYLOR[1:]:
        p = (p * r).astype(np.float32)
        p = (p + c).astype(np.float32)
    with np.errstate(over="ignore"):
        y = np.ldexp(p, n.astype(np.int32)).astype(np.float32)
    return np.where(nan, _F(np.nan), y).astype(np.float32)


def silu_f32(g) -> np.ndarray:
    """fp32 g / (1 + exp(-g)) (one add, one IEEE division)."""
    g = np.asarray(g, np.float32)
    d = (_F(1.0) + exp_f32(-g)).astype(np.float32)
    with np.errstate(invalid="ignore"):
        return (g / d).astype(np.float32)


def swiglu_bf16(h) -> np.ndarray:
    """Activation [M, F] (bf16 values as float64) of a gate/up output h
    [M, 2F] given as float values (bf16-representable)."""
    h = np.asarray(h, np.float32)
    F = h.shape[-1] // 2
    g, u = h[..., :F], h[..., F:]
    with np.errstate(invalid="ignore", over="ignore"):
        a = (silu_f32(g) * u).astype(np.float32)
    return round_bf16(a.astype(np.float64))
