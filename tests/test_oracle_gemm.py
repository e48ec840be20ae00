"""Pins of the grouped-GEMM oracle (CPU only).

Pinned against: pure-Python brute force on tiny ragged shapes (with its own
per-element dequantization from the unit definitions), exact integer
arithmetic, a gather-based formulation of the grouped product, the
per-128-block promotion form of blockwise scaling, the bf16 rounding
definition, the SQNR closed form of a uniform rounding error, and
structural facts (empty groups, expert permutation).
"""
import math

import numpy as np
import pytest

from oracle import formats as F
from oracle import quant as Q
from oracle import gemm as G
from mx_scaled_grouped_amd import workloads as W


def _unit_scale_act(q, recipe, r, c, layout="row"):
    """Scale of element (r, c) of a row-wise token tensor, by the unit definition."""
    sc = q["row_scales"] if layout == "row" else q["col_scales"]
    if recipe in ("tw", "dl"):
        return float(sc[0])
    if recipe == "block":
        return float(sc[r][c // 128])
    if recipe == "nvfp4":
        return F.decode_value(F.E4M3, int(sc[r][c // 16])) * float(q["tensor_scale"][0])
    return 2.0 ** (int(sc[r][c // 32]) - 127)


def _unit_scale_w(q, recipe, e, k, n, layout):
    if recipe in ("tw", "dl"):
        return float(q["kmajor_scales"][e])
    if recipe == "block":
        return float(q["kmajor_scales"][e][k // 128][n // 128])
    if recipe == "nvfp4":
        b = q["kmajor_scales"][e][n][k // 16] if layout == "k" else q["nmajor_scales"][e][k][n // 16]
        return F.decode_value(F.E4M3, int(b)) * float(q["tensor_scale"][e])
    if layout == "k":
        return 2.0 ** (int(q["kmajor_scales"][e][n][k // 32]) - 127)
    return 2.0 ** (int(q["nmajor_scales"][e][k][n // 32]) - 127)


def _sc(q, key, recipe):
    """The scales argument of the oracle's dequantization (nvfp4: block codes
    and the tensor scale)."""
    return (q[key], q["tensor_scale"]) if recipe == "nvfp4" else q[key]


@pytest.mark.parametrize("recipe,fa,fg", [("tw", F.E4M3, F.E5M2), ("block", F.E4M3, F.E4M3),
                                          ("mx", F.E4M3, F.E4M3), ("mx", F.E2M1, F.E2M1),
                                          ("nvfp4", F.E2M1, F.E2M1)],
                         ids=["tw", "block", "mx", "mxfp4", "nvfp4"])
def test_brute_force_tiny(recipe, fa, fg):
    """Forward, dgrad and wgrad of E=3, m = {0, 5, 13}, K=N=128 by triple loops."""
    sizes = [0, 5, 13]
    K, N = 128, 128
    a, w, dy, ge = W.small_case(21, sizes, K, N, outlier=True)
    qa = Q.quantize_act(a, recipe, fa, ge, rowwise=True, colwise=True)
    qd = Q.quantize_act(dy, recipe, fg, ge, rowwise=True, colwise=True)
    qw = Q.quantize_weight(w, recipe, fa)
    dec = lambda fmt, c: F.decode_value(fmt, int(c))
    st = Q.group_starts(ge)
    R = int(ge[-1])
    group_of = [g for g, m in enumerate(sizes) for _ in range(m)]

    def A(r, k):
        return dec(fa, qa["row_codes"][r][k]) * _unit_scale_act(qa, recipe, r, k)

    def D(r, n):
        return dec(fg, qd["row_codes"][r][n]) * _unit_scale_act(qd, recipe, r, n)

    def Wk(e, k, n):   # forward operand, from the k-major codes [E, N, K]
        return dec(fa, qw["kmajor_codes"][e][n][k]) * _unit_scale_w(qw, recipe, e, k, n, "k")

    def Wn(e, k, n):   # dgrad operand, from the n-major codes [E, K, N]
        return dec(fa, qw["nmajor_codes"][e][k][n]) * _unit_scale_w(qw, recipe, e, k, n, "n")

    Aq = [[A(r, k) for k in range(K)] for r in range(R)]
    Dq = [[D(r, n) for n in range(N)] for r in range(R)]
    E = len(sizes)
    Wkq = [[[Wk(e, k, n) for n in range(N)] for k in range(K)] for e in range(E)]
    Wnq = [[[Wn(e, k, n) for n in range(N)] for k in range(K)] for e in range(E)]

    # forward
    Y = G.grouped_fwd(G.deq_act_rows(qa["row_codes"], _sc(qa, "row_scales", recipe), recipe, fa),
                      G.deq_weight(qw, recipe, fa, "k"), ge)
    for r in range(R):
        g = group_of[r]
        for n in range(0, N, 7):
            want = math.fsum(Aq[r][k] * Wkq[g][k][n] for k in range(K))
            assert abs(Y[r, n] - want) <= 1e-12 * (abs(want) + 1e-30), (r, n)
    # dgrad
    dA = G.grouped_dgrad(G.deq_act_rows(qd["row_codes"], _sc(qd, "row_scales", recipe), recipe, fg),
                         G.deq_weight(qw, recipe, fa, "n"), ge)
    for r in range(R):
        g = group_of[r]
        for k in range(0, K, 5):
            want = math.fsum(Dq[r][n] * Wnq[g][k][n] for n in range(N))
            assert abs(dA[r, k] - want) <= 1e-12 * (abs(want) + 1e-30), (r, k)
    # wgrad from the column-wise (padded, transposed) operands
    At = G.unpad_cols(G.deq_act_cols(qa["col_codes"], _sc(qa, "col_scales", recipe), recipe, fa),
                      qa["padded_starts"], ge)
    Dt = G.unpad_cols(G.deq_act_cols(qd["col_codes"], _sc(qd, "col_scales", recipe), recipe, fg),
                      qd["padded_starts"], ge)
    dW = G.grouped_wgrad(At, Dt, ge, E)
    for e in range(E):
        rows = range(st[e], st[e] + sizes[e])
        for k in range(0, K, 9):
            for n in range(0, N, 11):
                # the column-wise operands of each row r, by the unit definition
                want = math.fsum(_col_val(qa, recipe, fa, e, r - st[e], k) * _col_val(qd, recipe, fg, e, r - st[e], n)
                                 for r in rows)
                assert abs(dW[e, k, n] - want) <= 1e-12 * (abs(want) + 1e-30), (e, k, n)
        if sizes[e] == 0:
            assert np.all(dW[e] == 0)


def _col_val(q, recipe, fmt, g, j, c):
    """Value of token j of group g, feature c, from the column-wise padded layout."""
    p = int(q["padded_starts"][g]) + j
    code = q["col_codes"][c][p]
    if recipe in ("tw", "dl"):
        s = float(q["col_scales"][0])
    elif recipe == "block":
        s = float(q["col_scales"][c][p // 128])
    elif recipe == "nvfp4":
        s = F.decode_value(F.E4M3, int(q["col_scales"][c][p // 16])) * float(q["tensor_scale"][0])
    else:
        s = 2.0 ** (int(q["col_scales"][c][p // 32]) - 127)
    return F.decode_value(fmt, int(code)) * s


def test_exact_integer_gemm():
    """Small-integer operands with power-of-two scales: every partial sum is an
    integer below 2^24, so the float64 oracle equals exact int64 arithmetic."""
    rng = np.random.default_rng(5)
    sizes = [0, 7, 130, 1, 64]
    R, K, N, E = sum(sizes), 256, 128, len(sizes)
    ge = W.group_ends_from_sizes(sizes)
    a = rng.integers(-8, 9, size=(R, K))
    w = rng.integers(-8, 9, size=(E, K, N))
    d = rng.integers(-8, 9, size=(R, N))
    Y = G.grouped_fwd(a * 0.5, w * 0.25, ge)
    dA = G.grouped_dgrad(d * 2.0, w * 0.25, ge)
    dW = G.grouped_wgrad(a * 0.5, d * 2.0, ge, E)
    st = Q.group_starts(ge)
    for g in range(E):
        sl = slice(st[g], ge[g])
        assert np.array_equal(Y[sl] * 8, (a[sl] @ w[g]).astype(np.float64))
        assert np.array_equal(dA[sl] * 2, (d[sl] @ w[g].T).astype(np.float64))
        assert np.array_equal(dW[g], (a[sl].T @ d[sl]).astype(np.float64))


def test_gather_formulation_and_one_group():
    """Grouped forward == a gather of each row's expert weight (no group loop);
    a single group is a plain GEMM."""
    sizes = [3, 0, 40, 17]
    a, w, dy, ge = W.small_case(22, sizes, 128, 256)
    af = Q.bf16_to_f32(a).astype(np.float64)
    wf = Q.bf16_to_f32(w).astype(np.float64)
    group_of = np.repeat(np.arange(len(sizes)), sizes)
    Y = G.grouped_fwd(af, wf, ge)
    Yg = np.einsum("rk,rkn->rn", af, wf[group_of])
    assert np.allclose(Y, Yg, rtol=1e-12, atol=1e-12)
    Y1 = G.grouped_fwd(af, wf[2:3], W.group_ends_from_sizes([sum(sizes)]))
    assert np.allclose(Y1, np.einsum("rk,kn->rn", af, wf[2]), rtol=1e-12, atol=1e-12)


def test_blockwise_promotion_form():
    """Dequantize-then-multiply equals the kernel-style form that sums raw code
    products per 128-wide contraction block and then scales by sA * sB."""
    sizes = [50, 130]
    K, N = 384, 256
    a, w, _, ge = W.small_case(23, sizes, K, N)
    qa = Q.quantize_act(a, "block", F.E4M3, ge)
    qw = Q.quantize_weight(w, "block", F.E4M3)
    Y = G.grouped_fwd(G.deq_act_rows(qa["row_codes"], qa["row_scales"], "block", F.E4M3),
                      G.deq_weight(qw, "block", F.E4M3, "k"), ge)
    va = F.decode(qa["row_codes"], F.E4M3)
    vw = F.decode(qw["kmajor_codes"], F.E4M3)             # [E, N, K]
    st = Q.group_starts(ge)
    for g in range(2):
        acc = np.zeros((sizes[g], N))
        for kb in range(K // 128):
            part = va[st[g]:ge[g], kb * 128:(kb + 1) * 128] @ vw[g, :, kb * 128:(kb + 1) * 128].T
            sA = qa["row_scales"][st[g]:ge[g], kb].astype(np.float64)[:, None]
            sB = np.repeat(qw["kmajor_scales"][g, kb, :].astype(np.float64), 128)[None, :]
            acc += part * sA * sB
        # the two forms differ only in float64 summation order
        assert np.max(np.abs(Y[st[g]:ge[g]] - acc)) <= 1e-12 * np.max(np.abs(acc))


def test_round_bf16_definition():
    """Nearest bf16 with ties to even, checked against bracketing by the bf16 grid."""
    rng = np.random.default_rng(9)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-40, 38, 20000),
                        [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 2.0 ** -133 * 1.5, 2.0 ** -133 * 2.5]])
    y = G.round_bf16(x)
    for xi, yi in zip(x[:3000].tolist() + x[-6:].tolist(), y[:3000].tolist() + y[-6:].tolist()):
        if xi == 0:
            assert yi == 0
            continue
        a = abs(xi)
        e = max(math.frexp(a)[1], -125)
        q = 2.0 ** (e - 8)                      # spacing of bf16 values around a
        lo = math.floor(a / q) * q
        hi = lo + q
        if a - lo < hi - a:
            want = lo
        elif a - lo > hi - a:
            want = hi
        else:
            want = lo if int(round(lo / q)) % 2 == 0 else hi
        assert abs(yi) == want and math.copysign(1, yi) == math.copysign(1, xi), (xi, yi, want)
    assert G.round_bf16(np.float64([1.0 + 2 ** -8]))[0] == 1.0
    assert G.round_bf16(np.float64([1.0 + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6


@pytest.mark.parametrize("fmt,want_db", [(F.E4M3, 31.5), (F.E5M2, 25.5)], ids=["e4m3", "e5m2"])
def test_sqnr_closed_form(fmt, want_db):
    """A relative rounding step of 2^-p (p mantissa bits) on log-uniform
    significands has relative error power 2^(-2p) * 3 / (96 ln 2), i.e.
    about 31.5 dB for e4m3 and 25.5 dB for e5m2; tensorwise quantization of
    N(0,1) data should land within 1 dB of it."""
    x = W.normal_bf16(31, 0, (512, 1024))
    q = Q.quantize_act(x, "tw", fmt)
    xq = G.deq_act_rows(q["row_codes"], q["row_scales"], "tw", fmt)
    p = fmt.man_bits
    pred = -10 * math.log10(2.0 ** (-2 * p) * 3 / (96 * math.log(2)))
    assert abs(pred - want_db) < 0.1
    got = G.sqnr_db(Q.bf16_to_f32(x), xq)
    assert abs(got - pred) < 1.0, (got, pred)


def test_structural_empty_group_and_permutation():
    sizes = [4, 0, 9]
    a, w, dy, ge = W.small_case(24, sizes, 128, 128)
    af = Q.bf16_to_f32(a).astype(np.float64)
    df = Q.bf16_to_f32(dy).astype(np.float64)
    wf = Q.bf16_to_f32(w).astype(np.float64)
    dW = G.grouped_wgrad(af, df, ge, 3)
    assert np.all(dW[1] == 0)
    init = np.full(dW.shape, 3.0)
    dW2 = G.grouped_wgrad(af, df, ge, 3, init=init)
    assert np.all(dW2[1] == 3.0)
    assert int(ge[-1]) == sum(sizes) == a.shape[0]
    # permute experts (2, 0, 1) together with their rows
    perm = [2, 0, 1]
    st = Q.group_starts(ge)
    rows = np.concatenate([np.arange(st[g], ge[g]) for g in perm])
    ge_p = W.group_ends_from_sizes([sizes[g] for g in perm])
    Y = G.grouped_fwd(af, wf, ge)
    Yp = G.grouped_fwd(af[rows], wf[perm], ge_p)
    assert np.array_equal(Yp, Y[rows])
    dWp = G.grouped_wgrad(af[rows], df[rows], ge_p, 3)
    assert np.array_equal(dWp, dW[perm])


def test_rel_fro_hand_cases():
    """||y - ref||_F / ||ref||_F on cases worked by hand: a 3-4-5 triangle
    (a missing square root gives 0.01 instead of 0.1, a swapped denominator
    0.5/||y|| instead of 0.5/||ref||), a matrix and a 3-D (weight-gradient
    shaped) array, and the zero conventions."""
    ref = np.array([[3.0, 0.0], [0.0, 4.0]])          # ||ref||_F = 5
    y = ref + np.array([[0.0, 0.5], [0.0, 0.0]])      # ||y - ref||_F = 0.5
    assert G.rel_fro(y, ref) == 0.1
    # the error is measured relative to the reference, not to y
    assert G.rel_fro(2 * ref, ref) == 1.0
    assert G.rel_fro(ref, 2 * ref) == 0.5
    # every element of a 3-D array counts: ||(1,2,2)|| = 3 over two experts
    ref3 = np.zeros((2, 2, 2))
    ref3[0, 0, 0], ref3[1, 1, 0], ref3[1, 1, 1] = 1.0, 2.0, 2.0
    y3 = ref3.copy()
    y3[1, 0, 1] = 0.75                                # error 0.75 -> 0.25
    assert G.rel_fro(y3, ref3) == 0.25
    assert G.rel_fro(np.zeros(3), np.zeros(3)) == 0.0
    assert G.rel_fro(np.ones(3), np.zeros(3)) == float("inf")


@pytest.mark.parametrize("k", [1, 7, 10, 23, 40])
def test_rel_fro_and_sqnr_power_of_two_perturbation(k):
    """ref * (1 + 2^-k) differs from ref by exactly ref * 2^-k (small
    integers, so every value is exact in float64), hence rel_fro is exactly
    2^-k and SQNR exactly 20 k log10(2) dB, whatever the shape or sign."""
    rng = np.random.default_rng(k)
    ref = rng.integers(-100, 101, size=(17, 9)).astype(np.float64)
    y = ref * (1.0 + 2.0 ** -k)
    assert G.rel_fro(y, ref) == 2.0 ** -k
    assert abs(G.sqnr_db(ref, y) - 20.0 * k * math.log10(2.0)) < 1e-9
    assert G.sqnr_db(ref, ref) == float("inf")
