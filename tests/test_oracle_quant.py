"""Pins of the quantization oracle (CPU only).

Each test checks the oracle against something other than itself: exact
rational arithmetic for the scale quotient, closed forms for the MX
exponent, scale equivariance, sign symmetry, the transpose identity of
the Transformer Engine design note (column-wise 128x1 == row-wise 1x128
of the transpose), the zero fill of partial blocks, the shape rule, and
the delayed-scaling closed form.
"""
from fractions import Fraction
import math

import numpy as np
import pytest

from oracle import formats as F
from oracle import quant as Q
from oracle.delayed import DelayedState
from mx_scaled_grouped_amd import workloads as W

FMTS = [F.E4M3, F.E5M2]
MX_FMTS = [F.E4M3, F.E5M2, F.E2M1]   # MX also carries the 4-bit e2m1 element (MXFP4)


def _f32_round_fraction(fr: Fraction) -> float:
    """Nearest float32 to an exact rational (ties to even), by bracketing."""
    x = np.float32(float(fr))          # within one ulp of the answer
    cands = [np.nextafter(x, np.float32(-np.inf)), x, np.nextafter(x, np.float32(np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - fr),
                                     int(np.float32(c).view(np.uint32)) & 1))
    return float(best)


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_scale_is_correctly_rounded_quotient(fmt):
    rng = np.random.default_rng(1)
    amax = np.abs(rng.standard_normal(300).astype(np.float32)) * np.float32(3.7)
    amax = np.concatenate([amax, np.float32([1.0, 448.0, 57344.0, 1e-20, 3e30, 0.1])])
    s, inv = Q.fp32_scale_pair(amax, fmt)
    for a, si, ii in zip(amax, s, inv):
        assert float(si) == _f32_round_fraction(Fraction(float(a)) / Fraction(fmt.fmax))
        assert float(ii) == _f32_round_fraction(Fraction(fmt.fmax) / Fraction(float(a)))
    s0, i0 = Q.fp32_scale_pair(np.float32(0), fmt)
    assert float(s0) == 1.0 and float(i0) == 1.0


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
@pytest.mark.parametrize("recipe", ["tw", "block"])
def test_amax_element_encodes_to_max(fmt, recipe):
    """The element that sets a unit's amax lands on +-fmax (x * fmax/amax rounds to fmax)."""
    x = W.normal_bf16(11, 0, (256, 512), std=3.0)
    q = Q.quantize_act(x, recipe, fmt)
    xf = Q.bf16_to_f32(x)
    if recipe == "tw":
        i = np.unravel_index(np.argmax(np.abs(xf)), xf.shape)
        assert q["row_codes"][i] & 0x7F == fmt.max_code
    else:
        blocks = np.abs(xf).reshape(256, 4, 128)
        j = np.argmax(blocks, axis=2)
        codes = q["row_codes"].reshape(256, 4, 128)
        picked = np.take_along_axis(codes, j[..., None], axis=2)[..., 0]
        assert np.all((picked & 0x7F) == fmt.max_code)
    assert np.all((q["row_codes"] & 0x7F) <= fmt.max_code)     # never NaN / Inf codes


def _mx_k_closed_form(a: float, fmt) -> int:
    """k = E - emax + [f > F] with a = f * 2^E, 1 <= f < 2 and fmax = F * 2^emax
    (F = 1.75 for e4m3 / e5m2, 1.5 for e2m1): the algebra of
    amax <= F * 2^(emax + k), clamped to [-127, 127]."""
    if a == 0:
        return 0
    m, e = math.frexp(a)          # a = m 2^e, 0.5 <= m < 1
    f, E = 2 * m, e - 1
    F_sig = {"e4m3": 1.75, "e5m2": 1.75, "e2m1": 1.5}[fmt.name]
    return max(-127, min(127, E - fmt.emax + (1 if f > F_sig else 0)))


@pytest.mark.parametrize("fmt", MX_FMTS, ids=lambda f: f.name)
def test_mx_exponent_edges(fmt):
    pts = [0.0]
    for j in range(-30, 30, 3):
        base = float(np.float32(fmt.fmax * 2.0 ** j))
        pts += [base, float(np.nextafter(np.float32(base), np.float32(np.inf))),
                float(np.nextafter(np.float32(base), np.float32(0))), 2.0 ** j,
                float(np.nextafter(np.float32(1.75 * 2 ** j), np.float32(np.inf))), 1.75 * 2 ** j]
    pts += [1e-45, 1e-40, 2.0 ** -140, 3.0e38]
    for a in pts:
        k = Q.mx_exponent(a, fmt)
        assert k == _mx_k_closed_form(a, fmt), a
        code = int(Q.mx_scale_codes(np.float32(a), fmt))
        assert code == k + 127
        if a > 0 and -127 < k < 127:
            assert a <= fmt.fmax * 2.0 ** k and a > fmt.fmax * 2.0 ** (k - 1)
    assert Q.mx_exponent(fmt.fmax * 2.0 ** 5, fmt) == 5
    assert Q.mx_exponent(2.0 ** -140, fmt) == -127


def test_mx_block_never_saturates():
    x = W.normal_bf16(12, 0, (64, 256), std=10.0)
    for fmt in MX_FMTS:
        q = Q.quantize_act(x, "mx", fmt)
        xf = Q.bf16_to_f32(x).reshape(64, 8, 32)
        inv = Q.mx_inv_from_codes(q["row_scales"])
        assert np.all(np.abs(xf * inv[..., None]) <= fmt.fmax)


def _all_outputs(x, recipe, fmt, ge):
    return Q.quantize_act(x, recipe, fmt, ge, rowwise=True, colwise=True,
                          dl_scale=(np.float32(0.25), np.float32(4.0)))


@pytest.mark.parametrize("recipe", ["tw", "block", "mx"])
@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_scale_equivariance(recipe, fmt):
    """quantize(2^j x): same codes, scales times 2^j (E8M0 code + j)."""
    x = W.normal_bf16(13, 0, (200, 256))
    ge = W.group_ends_from_sizes([70, 0, 129, 1])
    q0 = _all_outputs(x, recipe, fmt, ge)
    xf = Q.bf16_to_f32(x)
    for j in (-20, -7, -1, 1, 3, 20):
        xs = W.bf16_bits(xf * np.float32(2.0 ** j))            # exact power-of-two scaling
        q1 = _all_outputs(xs, recipe, fmt, ge)
        for key in ("row_codes", "col_codes"):
            assert np.array_equal(q0[key], q1[key]), (key, j)
        for key in ("row_scales", "col_scales"):
            if recipe == "mx":
                a0 = q0[key].astype(int)
                a1 = q1[key].astype(int)
                # all-padding blocks (amax 0) keep code 127
                assert np.all((a1 == a0 + j) | ((a0 == 127) & (a1 == 127))), (key, j)
            else:
                assert np.array_equal(q1[key], (q0[key] * np.float32(2.0 ** j)).astype(np.float32)), (key, j)


@pytest.mark.parametrize("recipe", ["tw", "block", "mx"])
def test_sign_symmetry(recipe):
    x = W.normal_bf16(14, 0, (150, 384))
    ge = W.group_ends_from_sizes([3, 147])
    q0 = _all_outputs(x, recipe, F.E4M3, ge)
    q1 = _all_outputs(x ^ np.uint16(0x8000), recipe, F.E4M3, ge)
    assert np.array_equal(q1["row_codes"], q0["row_codes"] ^ 0x80)
    P = q0["padded_starts"]
    for g, (a, b) in enumerate(zip(Q.group_starts(ge), ge)):
        sl = slice(P[g], P[g] + (b - a))
        assert np.array_equal(q1["col_codes"][:, sl], q0["col_codes"][:, sl] ^ 0x80)
    assert np.array_equal(q1["row_scales"], q0["row_scales"])
    assert np.array_equal(q1["col_scales"], q0["col_scales"])


@pytest.mark.parametrize("recipe", ["block", "mx", "tw"])
@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: f.name)
def test_transpose_identity(recipe, fmt):
    """Column-wise codes of group g == row-wise codes of x_g^T zero-padded to a
    multiple of 128 (transpose(bs_128x1(x)) == bs_1x128(transpose(x)))."""
    sizes = [0, 1, 31, 33, 127, 128, 129, 257, 0]
    x, _, _, ge = W.small_case(3, sizes, 256, 128)
    q = Q.quantize_act(x, recipe, fmt, ge, rowwise=True, colwise=True)
    P = q["padded_starts"]
    st = Q.group_starts(ge)
    blk = 32 if recipe == "mx" else 128
    assert P[-1] == sum(-(-m // 128) * 128 for m in sizes)
    for g, m in enumerate(sizes):
        mp = P[g + 1] - P[g]
        xt = np.zeros((256, mp), np.uint16)
        xt[:, :m] = x[st[g]:st[g] + m].T
        if mp == 0:
            continue
        if recipe == "tw":
            # one unit for the whole tensor: the column codes are the row codes moved
            assert np.array_equal(q["col_codes"][:, P[g]:P[g] + m], q["row_codes"][st[g]:st[g] + m].T)
            assert np.all(q["col_codes"][:, P[g] + m:P[g + 1]] == 0)
            continue
        r = Q.quantize_act(xt, recipe, fmt)          # row-wise 1xblk along the padded tokens
        assert np.array_equal(q["col_codes"][:, P[g]:P[g + 1]], r["row_codes"])
        assert np.array_equal(q["col_scales"][:, P[g] // blk:P[g + 1] // blk], r["row_scales"])


def test_zero_fill_partial_block():
    """A group of 5 rows: its 128x1 units are taken over the 5 rows present, and
    the 123 padding columns hold code 0x00 (the automatic zero fill)."""
    x, _, _, ge = W.small_case(4, [5, 130], 128, 128)
    q = Q.quantize_act(x, "block", F.E4M3, ge, rowwise=False, colwise=True)
    assert q["padded_starts"].tolist() == [0, 128, 384]
    xf = Q.bf16_to_f32(x)
    am = np.max(np.abs(xf[:5]), axis=0)
    s, _ = Q.fp32_scale_pair(am, F.E4M3)
    assert np.array_equal(q["col_scales"][:, 0], s)
    assert np.all(q["col_codes"][:, 5:128] == 0)
    assert np.all(q["col_codes"][:, 128 + 130:] == 0)
    # padding a block with zeros explicitly changes nothing
    xpad = np.zeros((128, 128), np.uint16)
    xpad[:5] = x[:5]
    r = Q.quantize_act(xpad.T.copy(), "block", F.E4M3)
    assert np.array_equal(r["row_codes"], q["col_codes"][:, :128])


def test_shape_rules():
    x = W.normal_bf16(15, 0, (130, 256))
    q = Q.quantize_act(x, "block", F.E4M3, W.group_ends_from_sizes([130]), colwise=True)
    assert q["row_scales"].shape == (130, 2)
    assert q["col_scales"].shape == (256, 2)            # 130 rows pad to 256 columns
    q = Q.quantize_act(x, "mx", F.E4M3, W.group_ends_from_sizes([130]), colwise=True)
    assert q["row_scales"].shape == (130, 8) and q["col_scales"].shape == (256, 8)
    w = W.normal_bf16(15, 1, (3, 256, 384), std=0.02)
    qw = Q.quantize_weight(w, "block", F.E4M3)
    assert qw["nmajor_scales"].shape == (3, 2, 3)
    qw = Q.quantize_weight(w, "mx", F.E4M3)
    assert qw["nmajor_scales"].shape == (3, 256, 12) and qw["kmajor_scales"].shape == (3, 384, 8)
    with pytest.raises(ValueError):
        Q.quantize_act(W.normal_bf16(15, 2, (16, 200)), "block", F.E4M3)
    with pytest.raises(ValueError):
        Q.quantize_weight(W.normal_bf16(15, 3, (1, 200, 128)), "tw", F.E4M3)


@pytest.mark.parametrize("recipe", ["dl", "block", "mx"])
def test_gather_row_equivariance(recipe):
    """Row-wise units never mix rows, so quantizing gathered rows equals
    gathering the rows of the quantized tensor (codes and per-row scales),
    for a permutation with repeats and tokens left out."""
    x = W.normal_bf16(16, 0, (40, 256))
    rng = np.random.default_rng(5)
    idx = rng.integers(0, 40, size=57)
    idx[:3] = [39, 0, 39]
    dl = (np.float32(0.01), np.float32(100.0))
    full = Q.quantize_act(x, recipe, F.E4M3, dl_scale=dl)
    g = Q.quantize_act_gather(x, idx, recipe, F.E4M3, dl_scale=dl)
    assert np.array_equal(g["row_codes"], full["row_codes"][idx])
    if recipe != "dl":
        assert np.array_equal(g["row_scales"], full["row_scales"][idx])


def test_gather_tensorwise_amax_over_routed_rows():
    """The tensorwise scale of a gathered operand comes from the routed rows:
    a token that no expert receives does not raise it."""
    x = W.normal_bf16(16, 1, (8, 128))
    big = np.float32(1000.0).view(np.uint32) >> 16
    x[5, 7] = big                       # the largest element sits in token 5
    idx = np.array([0, 1, 2, 3, 4, 6, 7, 0], np.int64)    # token 5 is dropped
    g = Q.quantize_act_gather(x, idx, "tw", F.E4M3)
    xf = Q.bf16_to_f32(x)
    want = np.max(np.abs(xf[[0, 1, 2, 3, 4, 6, 7]]))
    assert g["amax"][0] == want and want < 1000.0
    assert Q.quantize_act(x, "tw", F.E4M3)["amax"][0] == np.float32(1000.0)
    with pytest.raises(ValueError):
        Q.gather_rows(x, [0, 8])


def test_gather_columnwise_follows_groups():
    """Column-wise output of gathered rows: group g's tokens in routed order
    at padded columns [P_g, P_g + m_g); an identity index reproduces the
    plain call."""
    x = W.normal_bf16(16, 2, (30, 128))
    ge = W.group_ends_from_sizes([7, 0, 23])
    ident = np.arange(30)
    a = Q.quantize_act_gather(x, ident, "mx", F.E4M3, ge, colwise=True)
    b = Q.quantize_act(x, "mx", F.E4M3, ge, colwise=True)
    for k in ("row_codes", "row_scales", "col_codes", "col_scales", "padded_starts"):
        assert np.array_equal(a[k], b[k]), k
    rev = ident[::-1].copy()
    c = Q.quantize_act_gather(x, rev, "block", F.E4M3, ge, colwise=True)
    # group 0 = routed rows 0..6 = tokens 29..23, in that order
    d = Q.quantize_act(x[23:30][::-1].copy(), "block", F.E4M3, W.group_ends_from_sizes([7]), colwise=True)
    assert np.array_equal(c["col_codes"][:, :7], d["col_codes"][:, :7])
    assert np.array_equal(c["col_scales"][:, 0], d["col_scales"][:, 0])


def test_weight_layouts_agree():
    """k-major codes are the transposed n-major codes for tw and 128x128 tiles;
    128x128 units: a tile's max element lands on fmax."""
    w = W.normal_bf16(16, 0, (2, 256, 384), std=0.02)
    for recipe in ("tw", "block"):
        q = Q.quantize_weight(w, recipe, F.E4M3)
        assert np.array_equal(q["kmajor_codes"], q["nmajor_codes"].transpose(0, 2, 1))
    q = Q.quantize_weight(w, "block", F.E4M3)
    t = np.abs(Q.bf16_to_f32(w)).reshape(2, 2, 128, 3, 128)
    c = q["nmajor_codes"].reshape(2, 2, 128, 3, 128)
    for e in range(2):
        for i in range(2):
            for j in range(3):
                r, cc = np.unravel_index(np.argmax(t[e, i, :, j, :]), (128, 128))
                assert c[e, i, r, j, cc] & 0x7F == 0x7E
    # MX: each code set's blocks follow its own contraction dim
    q = Q.quantize_weight(w, "mx", F.E4M3)
    r = Q.quantize_act(w.reshape(-1, 384), "mx", F.E4M3)
    assert np.array_equal(r["row_codes"].reshape(2, 256, 384), q["nmajor_codes"])
    wT = np.ascontiguousarray(w.transpose(0, 2, 1)).reshape(-1, 256)
    r = Q.quantize_act(wT, "mx", F.E4M3)
    assert np.array_equal(r["row_codes"].reshape(2, 384, 256), q["kmajor_codes"])


def test_delayed_closed_form():
    """With amax growing 1.01x per step, s_t = max_{tau<t} amax_tau / fmax, s_0 = 1."""
    st = DelayedState(2, F.E4M3, history_len=1024)
    amaxes = [np.float32([3.0 * 1.01 ** t, 0.5]) for t in range(50)]
    assert st.scale(0) == (1.0, 1.0)
    for t, a in enumerate(amaxes):
        if t > 0:
            want = max(float(x[0]) for x in amaxes[:t])
            s, inv = st.scale(0)
            assert float(s) == _f32_round_fraction(Fraction(want) / Fraction(448))
            assert float(inv) == _f32_round_fraction(Fraction(448) / Fraction(want))
        st.update(a)


def test_delayed_window_expiry_and_guard():
    st = DelayedState(1, F.E5M2, history_len=4)
    seq = [8.0, 1.0, 1.0, 1.0, 1.0, 2.0]
    seen = []
    for a in seq:
        st.update([a])
        seen.append(float(st.s[0]))
    f = 57344.0
    assert seen == [float(np.float32(8 / f))] * 4 + [float(np.float32(1 / f)), float(np.float32(2 / f))]
    before = (float(st.s[0]), float(st.inv[0]))
    st2 = DelayedState(1, F.E5M2, history_len=2)
    st2.update([0.0])
    assert (float(st2.s[0]), float(st2.inv[0])) == (1.0, 1.0)      # a* == 0 keeps the previous scale
    st.update([np.inf])
    assert (float(st.s[0]), float(st.inv[0])) == before             # non-finite keeps it too


def test_delayed_saturation_count():
    """Under delayed scaling the saturated elements at step t >= 1 are those with
    |x_t| * inv_t > fmax (x drifts upward, so the newest max exceeds the history)."""
    st = DelayedState(1, F.E4M3)
    for t in range(4):
        x = W.normal_bf16(17, 0, (64, 128), std=1.01 ** (10 * t), step=t)
        s, inv = st.scale(0)
        q = Q.quantize_act(x, "dl", F.E4M3, dl_scale=(s, inv))
        xf = Q.bf16_to_f32(x)
        n_sat = int(np.sum((q["row_codes"] & 0x7F) == 0x7E))
        over = int(np.sum(np.abs((xf * inv).astype(np.float32)) > 448))
        at = int(np.sum(np.abs((xf * inv).astype(np.float32)) >= 464))   # rounds past max
        if t >= 1:
            assert n_sat >= over >= at
        st.update(q["amax"])


def test_amax_of_bf16_bits_matches_amax_of_values():
    """The bit-pattern amax equals max |x| of the widened values, including
    subnormals, signed zeros, the largest finite bf16 and chunk edges."""
    rng = np.random.default_rng(12)
    for n, chunk in ((1, 4), (1000, 7), (4096, 1 << 24)):
        x = rng.standard_normal(n).astype(np.float32) * np.float32(10.0) ** rng.integers(-40, 38, n).astype(np.float32)
        b = W.bf16_bits(np.nan_to_num(x, posinf=1e38, neginf=-1e38))
        assert Q.amax_of_bf16_bits(b, chunk) == Q.amax_of(Q.bf16_to_f32(b))
    special = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x7F7F, 0xFF7F, 0x3F80], np.uint16)
    assert Q.amax_of_bf16_bits(special) == Q.amax_of(Q.bf16_to_f32(special)) == Q.bf16_to_f32(np.uint16(0x7F7F))
    assert Q.amax_of_bf16_bits(np.array([0x8000, 0x0000], np.uint16)) == 0
