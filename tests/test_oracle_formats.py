"""Pins of the oracle's FP8 / E8M0 tables and its encoder (CPU only).

Pinned against: the OCP format standards' printed encodings (golden
fixture), the exhaustive 256-code round trip, and a brute-force nearest
code search that shares nothing with the oracle's table search.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ofp8_spec_points.json")


def _parse(v: str) -> float:
    v = v.strip()
    if v == "nan":
        return math.nan
    if v in ("inf", "-inf"):
        return math.copysign(math.inf, -1.0 if v.startswith("-") else 1.0)
    if v == "-0":
        return -0.0
    sign = -1.0 if v.startswith("-") else 1.0
    v = v.lstrip("-")
    val = 1.0
    for part in v.split("*"):
        if part.startswith("2^"):
            val *= 2.0 ** int(part[2:])
        else:
            val *= float(part)
    return sign * val


@pytest.mark.parametrize("name", ["e4m3", "e5m2", "e2m1"])
def test_spec_points(name):
    g = json.load(open(GOLDEN))
    fmt = F.FORMATS[name]
    assert g[name]["bias"] == fmt.bias
    t = F.decode_table(fmt)
    for code, val in g[name]["points"]:
        want = _parse(val)
        got = t[int(code, 16)]
        if math.isnan(want):
            assert math.isnan(got), (name, code)
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), (name, code, got, want)
    assert fmt.fmax == {"e4m3": 448.0, "e5m2": 57344.0, "e2m1": 6.0}[name]
    assert fmt.fmax == {"e4m3": 1.75, "e5m2": 1.75, "e2m1": 1.5}[name] * 2.0 ** fmt.emax


def test_e8m0_points():
    g = json.load(open(GOLDEN))
    for code, val in g["e8m0"]["points"]:
        want = _parse(val)
        got = float(F.e8m0_value(int(code, 16)))
        assert (math.isnan(want) and math.isnan(got)) or got == want


@pytest.mark.parametrize("name", ["e4m3", "e5m2", "e2m1"])
def test_roundtrip_all_codes(name):
    """decode -> encode is the identity on every finite code, including +-0."""
    fmt = F.FORMATS[name]
    t = F.decode_table(fmt)
    codes = np.arange(1 << fmt.bits)
    finite = np.isfinite(t)
    assert finite.sum() == {"e4m3": 254, "e5m2": 248, "e2m1": 16}[name]
    vals = t[finite].astype(np.float32)
    # -0.0 keeps its sign through float32
    vals[codes[finite] == fmt.sign_bit] = np.float32(-0.0)
    back = F.encode_sat_rne(vals, fmt)
    assert np.array_equal(back, codes[finite].astype(np.uint8))
    if fmt.ieee_specials:
        assert F.encode_sat_rne(np.float32([np.inf, -np.inf]), fmt).tolist() == [0x7B, 0xFB]
    # positive finite values strictly increase with the code
    pos = t[: fmt.max_code + 1]
    assert np.all(np.diff(pos) > 0)


def _brute_force_encode(v: np.ndarray, fmt) -> np.ndarray:
    """Nearest finite code by exhaustive distance to every code; ties to the
    even code; saturating; sign from the sign bit (independent of the oracle)."""
    vals = np.array([F.decode_value(fmt, c) for c in range(1 << fmt.bits)])
    half = 1 << (fmt.bits - 1)
    cand = np.array([c for c in range(half) if np.isfinite(vals[c])])     # non-negative codes
    a = np.abs(v.astype(np.float64))
    a = np.minimum(a, vals[fmt.max_code])                                  # saturate
    d = np.abs(a[:, None] - vals[cand][None, :])
    best = d.min(axis=1, keepdims=True)
    tie_ok = d == best
    # among the nearest, prefer even codes, then the smaller one
    score = np.where(tie_ok, (cand[None, :] & 1) * 1000 + cand[None, :], 10 ** 9)
    code = cand[np.argmin(score, axis=1)]
    return (code | np.where(np.signbit(v), half, 0)).astype(np.uint8)


@pytest.mark.parametrize("name", ["e4m3", "e5m2", "e2m1"])
def test_encoder_all_bf16_inputs(name):
    """Every bf16 bit pattern (as an fp32 value) encodes like the brute force."""
    fmt = F.FORMATS[name]
    b = np.arange(1 << 16, dtype=np.uint32)
    v = (b << 16).view(np.float32)
    v = v[~np.isnan(v) & np.isfinite(v)]
    for chunk in np.array_split(v, 8):
        assert np.array_equal(F.encode_sat_rne(chunk, fmt), _brute_force_encode(chunk, fmt))


@pytest.mark.parametrize("name", ["e4m3", "e5m2", "e2m1"])
def test_encoder_midpoints_and_neighbours(name):
    """Every midpoint between adjacent codes goes to the even code; one fp32
    ulp either side goes to the nearer code; (max, inf) saturates."""
    fmt = F.FORMATS[name]
    t = F.decode_table(fmt)
    pos = t[: fmt.max_code + 1]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (pos[:-1] + pos[1:]) / 2)   # exact in fp32
    lo = np.arange(fmt.max_code)
    hi = lo + 1
    got = F.encode_sat_rne(mids, fmt)
    want = np.where(lo % 2 == 0, lo, hi)
    assert np.array_equal(got, want.astype(np.uint8))
    below = np.nextafter(mids, np.float32(-np.inf))
    above = np.nextafter(mids, np.float32(np.inf))
    assert np.array_equal(F.encode_sat_rne(below, fmt), lo.astype(np.uint8))
    assert np.array_equal(F.encode_sat_rne(above, fmt), hi.astype(np.uint8))
    assert np.array_equal(F.encode_sat_rne(-mids, fmt), (want | fmt.sign_bit).astype(np.uint8))
    big = np.float32([fmt.fmax * 1.0001, fmt.fmax * 2, 3.0e38, np.float32(fmt.fmax) + np.float32(8)])
    assert np.all(F.encode_sat_rne(big, fmt) == fmt.max_code)
    assert np.all(F.encode_sat_rne(-big, fmt) == fmt.max_code | fmt.sign_bit)


@pytest.mark.parametrize("name", ["e4m3", "e5m2", "e2m1"])
def test_encoder_random_fp32(name):
    """Random fp32 bit patterns over the finite range vs the brute force."""
    fmt = F.FORMATS[name]
    rng = np.random.default_rng(7)
    u = rng.integers(0, 1 << 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    v = u.view(np.float32)
    v = v[np.isfinite(v)]
    # also dense near the format's range
    w = (rng.standard_normal(100_000) * fmt.fmax / 4).astype(np.float32)
    for arr in (v, w):
        for chunk in np.array_split(arr, 10):
            assert np.array_equal(F.encode_sat_rne(chunk, fmt), _brute_force_encode(chunk, fmt))


def test_signed_zero_and_underflow():
    for fmt in (F.E4M3, F.E5M2, F.E2M1):
        tiny = np.float32([0.0, -0.0, 1e-30, -1e-30, 1e-45, -1e-45])
        sb = fmt.sign_bit
        assert F.encode_sat_rne(tiny, fmt).tolist() == [0, sb, 0, sb, 0, sb]


def test_nibble_packing():
    """Element 2i in the low nibble, 2i+1 in the high nibble; round trip."""
    c = np.array([[0x1, 0xF, 0x0, 0x8, 0x7, 0x2]], np.uint8)
    p = F.pack_nibbles(c)
    assert p.tolist() == [[0xF1, 0x80, 0x27]]
    assert np.array_equal(F.unpack_nibbles(p), c)
    r = np.random.default_rng(3).integers(0, 16, size=(5, 64)).astype(np.uint8)
    assert np.array_equal(F.unpack_nibbles(F.pack_nibbles(r)), r)
    with pytest.raises(ValueError):
        F.pack_nibbles(np.array([1, 2, 3], np.uint8))
    with pytest.raises(ValueError):
        F.encode_sat_rne(np.float32([np.nan]), F.E4M3)
