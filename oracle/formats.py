"""FP8 and E8M0 formats, built from their bit-field definitions.

The pages name the formats only: ``fp8="e4m3"`` in the coverage table of
the Megatron-LM single-grouped-weight PR, ``--fp8-format hybrid`` (e4m3
forward tensors, e5m2 gradients) in the Megatron-LM FP8-vs-BF16 bug
report's reproduction steps, and MXFP8 in the same PR's table. The field
definitions below are those of the OCP 8-bit floating point (OFP8) and
OCP Microscaling (MX) v1.0 specifications:

* e4m3: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities;
  S.1111.111 is NaN; the largest finite magnitude is 448 (0x7E).
* e5m2: 1 sign, 5 exponent (bias 15), 2 mantissa bits; S.11111.00 is
  +-Inf, S.11111.{01,10,11} are NaN; the largest finite is 57344 (0x7B).
* E8M0: an 8-bit biased exponent (bias 127): code c means 2^(c-127) for
  c in 0..254, and 255 is NaN.
* e2m1 (the MXFP4 element of OCP MX v1.0): 1 sign, 2 exponent (bias 1),
  1 mantissa bit, 4 bits in all; every code is finite; magnitudes
  0, 0.5, 1, 1.5, 2, 3, 4, 6. The Megatron-LM single-grouped-weight PR
  names fp4 primary weights and NVFP4 next to MXFP8; MXFP4 is the FP4
  variant with the same 32-element E8M0 blocks as MXFP8.

Test infrastructure; see the package docstring.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Fp8Format:
    """A small float format (8-bit unless ``bits`` says otherwise)."""
    name: str
    exp_bits: int
    man_bits: int
    bias: int
    ieee_specials: bool   # True: all-ones exponent is Inf/NaN (e5m2); False: only S.1111.111 is NaN
    bits: int = 8
    finite_only: bool = False   # no Inf / NaN codes at all (e2m1)

    @property
    def sign_bit(self) -> int:
        return 1 << (self.bits - 1)

    @property
    def max_code(self) -> int:
        """Largest positive finite code."""
        if self.finite_only:
            return self.sign_bit - 1
        return 0x7B if self.ieee_specials else 0x7E

    @property
    def fmax(self) -> float:
        return float(decode_table(self)[self.max_code])

    @property
    def emax(self) -> int:
        """Exponent of the largest finite value."""
        top = 2 ** self.exp_bits - (2 if self.ieee_specials else 1)
        return top - self.bias


E4M3 = Fp8Format("e4m3", 4, 3, 7, False)
E5M2 = Fp8Format("e5m2", 5, 2, 15, True)
E2M1 = Fp8Format("e2m1", 2, 1, 1, False, bits=4, finite_only=True)
FORMATS = {"e4m3": E4M3, "e5m2": E5M2, "e2m1": E2M1}

_TABLES = {}


def decode_value(fmt: Fp8Format, code: int) -> float:
    """Value of one code, from the sign / exponent / mantissa fields."""
    sign = -1.0 if (code >> (fmt.bits - 1)) & 1 else 1.0
    e = (code >> fmt.man_bits) & ((1 << fmt.exp_bits) - 1)
    m = code & ((1 << fmt.man_bits) - 1)
    e_all_ones = e == (1 << fmt.exp_bits) - 1
    if fmt.finite_only:
        pass
    elif fmt.ieee_specials and e_all_ones:
        return sign * math.inf if m == 0 else math.nan
    elif e_all_ones and m == (1 << fmt.man_bits) - 1:
        return math.nan
    if e == 0:   # subnormal: m * 2^(1 - bias - man_bits)
        return sign * math.ldexp(m, 1 - fmt.bias - fmt.man_bits)
    return sign * math.ldexp((1 << fmt.man_bits) + m, e - fmt.bias - fmt.man_bits)


def decode_table(fmt: Fp8Format) -> np.ndarray:
    """float64 [2^bits]: the value of every code (NaN codes give NaN)."""
    t = _TABLES.get(fmt.name)
    if t is None:
        t = np.array([decode_value(fmt, c) for c in range(1 << fmt.bits)], dtype=np.float64)
        t.setflags(write=False)
        _TABLES[fmt.name] = t
    return t


def encode_sat_rne(v, fmt: Fp8Format) -> np.ndarray:
    """Saturating round-to-nearest-even encode of float32 values to codes.

    The nearest finite code is found by searching the sorted table of
    non-negative finite values; a value exactly half-way between two codes
    takes the one whose least significant bit is 0; magnitudes above the
    largest finite value (including e5m2 +-Inf inputs) give +-max. The sign
    comes from the sign bit of the input, so -0 and negative values that
    round to zero give the sign bit alone (0x80; 0x8 for e2m1). NaN inputs
    are outside the contract. Codes are returned one per uint8.
    """
    v = np.asarray(v, dtype=np.float32)
    if np.isnan(v).any():
        raise ValueError("NaN input to the FP8 encoder")
    table = decode_table(fmt)
    pos = table[: fmt.max_code + 1]              # codes 0..max, increasing values
    a = np.abs(v.astype(np.float64))
    hi = np.searchsorted(pos, a, side="left")   # first code with value >= a
    hi = np.minimum(hi, fmt.max_code)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - pos[lo]
    d_hi = pos[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((hi & 1) == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= pos[fmt.max_code], fmt.max_code, code)   # saturate (and exact max)
    code = np.where(a == 0.0, 0, code)
    sign = np.signbit(v)
    return (code | np.where(sign, fmt.sign_bit, 0)).astype(np.uint8)


def decode(codes, fmt: Fp8Format) -> np.ndarray:
    """float64 values of an array of codes (one code per uint8)."""
    return decode_table(fmt)[np.asarray(codes, dtype=np.uint8)]


def pack_nibbles(codes) -> np.ndarray:
    """4-bit codes [..., L] (L even, one per uint8) -> bytes [..., L/2]:
    element 2i in the low nibble of byte i, element 2i+1 in the high one."""
    c = np.asarray(codes, dtype=np.uint8)
    if c.shape[-1] % 2 or (c > 0xF).any():
        raise ValueError("need an even count of 4-bit codes")
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed) -> np.ndarray:
    """Inverse of pack_nibbles."""
    b = np.asarray(packed, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


# ---- E8M0 (OCP MX v1.0 shared scale) -------------------------------------

E8M0_BIAS = 127
E8M0_NAN = 255


def e8m0_value(code) -> np.ndarray:
    c = np.asarray(code, dtype=np.int64)
    out = np.ldexp(1.0, c - E8M0_BIAS).astype(np.float64)
    return np.where(c == E8M0_NAN, np.nan, out)
