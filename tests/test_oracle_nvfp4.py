"""Pins of the NVFP4 oracle (oracle/quant.py: e2m1 elements, an e4m3 scale
per 16 elements along the contraction dim, an fp32 scale per tensor):
a worked example, power-of-two equivariance, sign symmetry, zeros,
element codes as the brute-force nearest grid points of x / (D s_t), and
the column-wise (16x1, per group) layout as the row-wise layout of the
transposed, zero-padded groups."""
import numpy as np
import pytest

from oracle import formats as F
from oracle import quant as Q
from oracle import gemm as G
from mx_scaled_grouped_amd import workloads as W


def _bits(vals):
    return W.bf16_bits(np.asarray(vals, np.float32))


def test_worked_example():
    """One row of 128 with three non-zero blocks (every value exact in bf16).
    Tensor amax 12: s_t = fp32(12 / 2688) = fp32(1/224) = 0.004464286.
    Block 0 (amax 12): t = fp32(2 / s_t) = 447.99997 -> e4m3 448 (0x7E);
      M = fp32(448 s_t) = 2, inv = 0.5: 12 -> 6 (0x7), -5 -> -2.5, a tie
      between 2 (index 4, even) and 3 -> 2 (0xC), 1.25 -> 0.625 -> 0.5 (0x1).
    Block 1 (amax 0.75): t = fp32(0.125 / s_t) = 27.999998 -> 28 (0x5E);
      M = 0.125, inv = 8: 0.75 -> 6 (0x7), 0.3125 -> 2.5 -> 2 (0x4),
      -0.0625 -> -0.5 (0x9), 0.01953125 -> 0.15625 -> 0 (0x0).
    Block 2 (amax 2^-7): t = fp32(fp32(2^-7 / 6) / s_t) = 0.29166666 ->
      e4m3 0.28125 (0x29; the other neighbour 0.3125 is farther);
      M = fp32(0.28125 s_t), 1 / M = 796.4445: 2^-7 -> 6.22 saturates to 6 (0x7).
    Blocks 3..7 are zero: code 0x00, element codes 0."""
    x = np.zeros(128, np.float32)
    x[[0, 1, 2]] = [12.0, -5.0, 1.25]
    x[[16, 17, 18, 19]] = [0.75, 0.3125, -0.0625, 0.01953125]
    x[32] = 2.0 ** -7
    q = Q.quantize_act(_bits(x).reshape(1, 128), "nvfp4", F.E2M1)
    assert q["tensor_scale"][0] == np.float32(12) / np.float32(2688)
    assert q["row_scales"][0].tolist() == [0x7E, 0x5E, 0x29, 0, 0, 0, 0, 0]
    c = q["row_codes"][0]
    assert c[[0, 1, 2]].tolist() == [0x7, 0xC, 0x1]
    assert c[[16, 17, 18, 19]].tolist() == [0x7, 0x4, 0x9, 0x0]
    assert c[32] == 0x7
    assert not c[np.setdiff1d(np.arange(128), [0, 1, 2, 16, 17, 18, 19, 32])].any()


@pytest.mark.parametrize("j", [-20, -3, 1, 7, 20])
def test_power_of_two_equivariance(j):
    x = W.normal_bf16(40, 0, (64, 256), std=3.0)
    q0 = Q.quantize_act(x, "nvfp4", F.E2M1)
    x2 = W.bf16_bits(Q.bf16_to_f32(x) * np.float32(2.0 ** j))
    q1 = Q.quantize_act(x2, "nvfp4", F.E2M1)
    assert np.array_equal(q0["row_codes"], q1["row_codes"])
    assert np.array_equal(q0["row_scales"], q1["row_scales"])
    assert q1["tensor_scale"][0] == np.float32(q0["tensor_scale"][0] * 2.0 ** j)


def test_sign_symmetry_and_zeros():
    x = W.normal_bf16(41, 0, (32, 128))
    q = Q.quantize_act(x, "nvfp4", F.E2M1)
    qn = Q.quantize_act(x ^ np.uint16(0x8000), "nvfp4", F.E2M1)
    assert np.array_equal(qn["row_codes"], q["row_codes"] ^ np.uint8(0x8))
    assert np.array_equal(qn["row_scales"], q["row_scales"])
    z = Q.quantize_act(np.zeros((3, 128), np.uint16), "nvfp4", F.E2M1)
    assert z["tensor_scale"][0] == 1.0 and not z["row_codes"].any() and not z["row_scales"].any()


def test_codes_are_nearest_grid_points():
    """Each code is the e2m1 value nearest to x * inv_b (ties to even,
    saturating at 6), found by a brute-force search over the 16 codes, with
    inv_b = fp32(1 / fp32(D s_t)) from the block code."""
    x = W.normal_bf16(42, 0, (16, 256), std=2.0)
    q = Q.quantize_act(x, "nvfp4", F.E2M1)
    xf = Q.bf16_to_f32(x)
    s_t = np.float32(q["tensor_scale"][0])
    vals = np.array([F.decode_value(F.E2M1, c) for c in range(16)])
    for r in range(16):
        for c in range(0, 256, 3):
            D = np.float32(F.decode_value(F.E4M3, int(q["row_scales"][r][c // 16])))
            inv = np.float32(1) / np.float32(D * s_t)
            v = float(np.float32(xf[r, c] * inv))
            v = max(-6.0, min(6.0, v))
            d = np.abs(vals - v)
            best = np.flatnonzero(d == d.min())
            if best.size > 1:                       # tie: the even code (mantissa bit 0)
                best = [b for b in best if b % 2 == 0 and (b >= 8) == (np.signbit(v))] or best
            got = int(q["row_codes"][r][c])
            assert vals[got] == vals[best[0]], (r, c, v, got, best)


def test_column_layout_is_rowwise_of_padded_transpose():
    sizes = [20, 0, 131, 16]
    x, _, _, ge = W.small_case(43, sizes, 128, 128)
    q = Q.quantize_act(x, "nvfp4", F.E2M1, ge, rowwise=True, colwise=True)
    P = q["padded_starts"]
    st = Q.group_starts(ge)
    for g, m in enumerate(sizes):
        xp = np.zeros(((m + 127) // 128 * 128, 128), np.uint16)
        xp[:m] = x[st[g]:st[g] + m]
        # row-wise blocks of the transposed, zero-padded group with the tensor's scale
        codes, sb = Q.nvfp4_blocks(Q.bf16_to_f32(xp.T).reshape(128, -1, 16), q["tensor_scale"][0])
        assert np.array_equal(q["col_codes"][:, P[g]:P[g + 1]], codes.reshape(128, -1))
        assert np.array_equal(q["col_scales"][:, P[g] // 16:P[g + 1] // 16], sb)


def test_weight_layouts_and_per_expert_scale():
    w = W.normal_bf16(44, 1, (3, 256, 128), std=0.02)
    w[1] = W.bf16_bits(Q.bf16_to_f32(w[1]) * np.float32(64))      # expert 1 larger by 2^6
    q = Q.quantize_weight(w, "nvfp4", F.E2M1)
    assert q["tensor_scale"][1] == np.float32(q["amax"][1] / np.float32(2688))
    for e in range(3):
        qe = Q.quantize_act(np.ascontiguousarray(w[e].T), "nvfp4", F.E2M1)    # rows = n, blocks along k
        assert np.array_equal(q["kmajor_codes"][e], qe["row_codes"])
        assert np.array_equal(q["kmajor_scales"][e], qe["row_scales"])
        qn = Q.quantize_act(w[e], "nvfp4", F.E2M1)                              # rows = k, blocks along n
        assert np.array_equal(q["nmajor_codes"][e], qn["row_codes"])
    Wd = G.deq_weight(q, "nvfp4", F.E2M1, "k")
    assert G.sqnr_db(Q.bf16_to_f32(w).astype(np.float64), Wd) > 18
