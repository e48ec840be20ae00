"""Quantization oracle: amax, scales, codes and layouts for every recipe.

Sources on the pages (none of them prints a formula):

* run-time quantization ahead of a scaled grouped matmul: the torchao
  float8 MoE training PR, Summary - each operand is quantized from the amax
  of the current tensor.
* delayed scaling with ``--fp8-amax-compute-algo max`` and
  ``--fp8-amax-history-len 1024``: the Megatron-LM FP8-vs-BF16 MoE bug
  report, reproduction steps (see ``delayed``).
* 1x128 scaling of forward activations, 128x1 scaling for backward with
  the transpose identity transpose(bs_128x1(x)) == bs_1x128(transpose(x)),
  and zero fill of a partial block: the Transformer Engine
  "FP8BlockQuantizer not work" issue, the maintainer's design note.
* the blocked feature dimension must be a multiple of 128 while the token
  dimension may be ragged: same issue, the shape rule and its correction.
* row-wise data, ``scale_inv``, column-wise data and column-wise
  ``scale_inv`` stored side by side for a grouped weight: the Megatron-LM
  single-grouped-weight PR, fix 1 (the MXFP8 GroupedTensor listing).
* MXFP8 with e4m3 elements: the same PR's coverage table.

Readings taken where the pages are silent:

* a scaling unit's scale is ``s = fp32(amax / fmax)`` (the stored
  dequantization multiplier, ``scale_inv`` in the PR's naming) and the
  cast multiplier is ``inv = fp32(fmax / amax)``, two independently
  rounded IEEE float32 divisions; amax == 0 gives s = inv = 1.
* a code is ``sat_rne(fp32(x * inv))``: the product is rounded to float32
  before encoding.
* MX: the E8M0 exponent k is the smallest integer with amax <= fmax * 2^k,
  clamped to [-127, 127] (k = 0 for amax == 0); s = 2^k, inv = 2^-k.
* tensorwise / delayed units: one per 2-D activation matrix, one per
  expert matrix of a 3-D weight.
* column-wise units of a token tensor restart at each expert group's first
  row; group g's tokens are placed at padded columns [P_g, P_g + m_g) with
  P_g = sum_{j<g} ceil(m_j / 128) * 128, and the gap up to P_{g+1} holds
  code 0x00. MX blocks that lie entirely in the gap get E8M0 code 127.

Test infrastructure; see the package docstring.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

from .formats import Fp8Format, encode_sat_rne, E8M0_BIAS

BLOCK = 128      # DeepSeek-style block length (the Transformer Engine issue's block size)
MX_BLOCK = 32    # MXFP8 block length (OCP MX v1.0)
NV_BLOCK = 16    # NVFP4 block length (16 e2m1 elements share an e4m3 scale)
NV_TENSOR_DEN = 2688.0   # 6 * 448: the largest e2m1 value times the largest e4m3 value
RECIPES = ("tw", "dl", "block", "mx", "nvfp4")


def bf16_to_f32(b) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact: bf16 is the top half of fp32)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---- scales -----------------------------------------------------------------

def amax_of(x_f32) -> np.float32:
    """max |x| over a unit; exact (no rounding is involved)."""
    x = np.asarray(x_f32, dtype=np.float32)
    if x.size == 0:
        return np.float32(0.0)
    return np.float32(np.max(np.abs(x)))


def amax_of_bf16_bits(bits, chunk: int = 1 << 24) -> np.float32:
    """max |x| over bf16 bit patterns of finite values, exactly, without
    widening to float32: a finite bf16 value's magnitude is ordered as its
    low 15 bits (exponent above mantissa), so the largest magnitude is the
    value of the largest masked pattern. Chunked, for tensors of billions of
    elements."""
    b = np.asarray(bits, np.uint16).reshape(-1)
    m = np.uint16(0)
    for i in range(0, b.size, chunk):
        m = max(m, np.max(b[i:i + chunk] & np.uint16(0x7FFF)))
    return np.float32(bf16_to_f32(np.array([m], np.uint16))[0])


def fp32_scale_pair(amax, fmt: Fp8Format):
    """(s, inv) as float32 for the fp32-scaled recipes: s = amax/fmax, inv = fmax/amax.

    Works element-wise on arrays. amax == 0 gives (1, 1).
    """
    a = np.asarray(amax, dtype=np.float32)
    fmax = np.float32(fmt.fmax)
    with np.errstate(divide="ignore", invalid="ignore"):
        s = np.where(a > 0, a / fmax, np.float32(1.0)).astype(np.float32)
        inv = np.where(a > 0, fmax / np.where(a > 0, a, np.float32(1.0)), np.float32(1.0)).astype(np.float32)
    if not np.all(np.isfinite(inv)):
        raise ValueError("amax too small: fmax/amax overflows float32 (outside the contract)")
    return s, inv


def mx_exponent(amax: float, fmt: Fp8Format) -> int:
    """Smallest integer k with amax <= fmax * 2^k, clamped to [-127, 127]; 0 for amax == 0."""
    a = float(amax)
    if a == 0.0:
        return 0
    k = math.ceil(math.log2(a / fmt.fmax))     # a first guess, then made exact
    while a > math.ldexp(fmt.fmax, k):
        k += 1
    while a <= math.ldexp(fmt.fmax, k - 1):
        k -= 1
    return max(-127, min(127, k))


def mx_scale_codes(amax, fmt: Fp8Format) -> np.ndarray:
    """E8M0 codes (k + 127) of an array of block amaxes (vectorized ``mx_exponent``)."""
    a = np.asarray(amax, dtype=np.float32).astype(np.float64)
    pos = a > 0
    safe = np.where(pos, a, 1.0)
    k = np.ceil(np.log2(safe / fmt.fmax)).astype(np.int64)        # a first guess, then made exact
    for _ in range(2):
        k = np.where(safe > np.ldexp(fmt.fmax, k), k + 1, k)
        k = np.where(safe <= np.ldexp(fmt.fmax, k - 1), k - 1, k)
    k = np.where(pos, np.clip(k, -127, 127), 0)
    return (k + E8M0_BIAS).astype(np.uint8)


def mx_inv_from_codes(codes) -> np.ndarray:
    """float32 2^-(c-127): exact for the codes a bf16 input can produce."""
    c = np.asarray(codes, dtype=np.int64)
    return np.ldexp(np.float32(1.0), -(c - E8M0_BIAS)).astype(np.float32)


def cast(x_f32, inv, fmt: Fp8Format) -> np.ndarray:
    """Codes of x with multiplier inv: sat_rne(fp32(x * inv)), no fused multiply-add."""
    prod = (np.asarray(x_f32, dtype=np.float32) * np.asarray(inv, dtype=np.float32)).astype(np.float32)
    return encode_sat_rne(prod, fmt)


# ---- NVFP4: e2m1 elements, e4m3 scale per 16 elements, fp32 scale per tensor ----
#
# The single-grouped-weight PR tests an NVFP4 recipe next to MXFP8 and MXFP4
# (coverage table: fp4 = e2m1 with the nvfp4 recipe). The pages give no
# formula; the reading taken (the two-level scheme of the public NVFP4
# format, each step one IEEE fp32 operation):
#   tensor unit (an activation tensor; one expert of a weight): amax_t,
#     s_t = fp32(amax_t / 2688), or 1 when amax_t == 0;
#   block of 16 consecutive elements along the contraction dim: amax_b,
#     t_b = fp32(fp32(amax_b / 6) / s_t), block code sb = e4m3 sat_rne(t_b),
#     D = value(sb), M_b = fp32(D * s_t), inv_b = fp32(1 / M_b) (0 when
#     M_b == 0 or 1 / M_b overflows);
#   element code q = e2m1 sat_rne(fp32(x * inv_b));
#   value: e2m1(q) * D * s_t (exact; the oracle dequantizes in float64).

def nvfp4_tensor_scale(amax) -> np.ndarray:
    """s_t = fp32(amax / 2688) per unit (1 for amax == 0)."""
    a = np.asarray(amax, np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.where(a > 0, a / np.float32(NV_TENSOR_DEN), np.float32(1.0)).astype(np.float32)


def nvfp4_blocks(xb, s_t):
    """Codes and e4m3 block codes of blocks along the last axis: xb float32
    [..., nb, 16] (zero-filled where a block is partial), s_t broadcastable
    to [..., nb]. Returns (codes u8 [..., nb, 16], block codes u8 [..., nb])."""
    from .formats import E4M3, E2M1, decode
    xb = np.asarray(xb, np.float32)
    am = np.max(np.abs(xb), axis=-1) if xb.shape[-1] else np.zeros(xb.shape[:-1], np.float32)
    s_t = np.asarray(s_t, np.float32)
    d6 = (am / np.float32(6.0)).astype(np.float32)
    t_b = (d6 / s_t).astype(np.float32)
    sb = encode_sat_rne(t_b, E4M3)
    D = decode(sb, E4M3).astype(np.float32)
    m_b = (D * s_t).astype(np.float32)
    with np.errstate(divide="ignore", over="ignore"):
        inv = np.where(m_b > 0, np.float32(1.0) / np.where(m_b > 0, m_b, np.float32(1.0)), np.float32(0.0))
    inv = np.where(np.isfinite(inv), inv, np.float32(0.0)).astype(np.float32)
    return cast(xb, inv[..., None], E2M1), sb


def _nvfp4_act(x, group_ends, rowwise, colwise, tensor_amax=None) -> dict:
    M, C = x.shape
    am = amax_of(x) if tensor_amax is None else np.float32(tensor_amax)
    s_t = nvfp4_tensor_scale(am)
    out = {"amax": np.array([am], np.float32), "tensor_scale": np.array([s_t], np.float32)}
    if rowwise:
        codes, sb = nvfp4_blocks(x.reshape(M, C // NV_BLOCK, NV_BLOCK), s_t)
        out["row_codes"] = codes.reshape(M, C)
        out["row_scales"] = sb
    if colwise:
        check_groups(group_ends, M)
        P = padded_starts(group_ends)
        st = group_starts(group_ends)
        ge = np.asarray(group_ends, dtype=np.int64)
        Rp = int(P[-1])
        xp = np.zeros((Rp, C), np.float32)                 # padded token layout, zero fill
        for g in range(len(P) - 1):
            m = int(ge[g] - st[g])
            xp[P[g]:P[g] + m] = x[st[g]:st[g] + m]
        # 16x1 blocks along the padded tokens; a group's first token starts a block
        codes, sb = nvfp4_blocks(xp.T.reshape(C, Rp // NV_BLOCK, NV_BLOCK), s_t)
        out["padded_starts"] = P
        out["col_codes"] = codes.reshape(C, Rp)
        out["col_scales"] = sb
    return out


def _nvfp4_weight(w, tensor_amax=None) -> dict:
    E, K, N = w.shape
    am = (np.array([amax_of(w[e]) for e in range(E)], np.float32) if tensor_amax is None
          else np.asarray(tensor_amax, np.float32).reshape(E))
    s_t = nvfp4_tensor_scale(am)
    cn, sn = nvfp4_blocks(w.reshape(E, K, N // NV_BLOCK, NV_BLOCK), s_t[:, None, None])
    wt = np.ascontiguousarray(w.transpose(0, 2, 1))                  # [E, N, K]
    ck, sk = nvfp4_blocks(wt.reshape(E, N, K // NV_BLOCK, NV_BLOCK), s_t[:, None, None])
    return {"amax": am, "tensor_scale": s_t,
            "nmajor_codes": cn.reshape(E, K, N), "nmajor_scales": sn,
            "kmajor_codes": ck.reshape(E, N, K), "kmajor_scales": sk}


# ---- group layout -----------------------------------------------------------

def group_starts(group_ends) -> np.ndarray:
    ge = np.asarray(group_ends, dtype=np.int64)
    return np.concatenate([[0], ge[:-1]]) if ge.size else np.zeros(0, np.int64)


def padded_starts(group_ends) -> np.ndarray:
    """int64 [E+1]: P_0 = 0, P_{g+1} = P_g + ceil(m_g / 128) * 128."""
    ge = np.asarray(group_ends, dtype=np.int64)
    m = ge - group_starts(ge)
    if np.any(m < 0):
        raise ValueError("group ends must be non-decreasing")
    pad = ((m + BLOCK - 1) // BLOCK) * BLOCK
    return np.concatenate([[0], np.cumsum(pad)]).astype(np.int64)


def check_groups(group_ends, M: int):
    ge = np.asarray(group_ends, dtype=np.int64)
    if ge.size == 0 or ge[-1] != M or np.any(np.diff(np.concatenate([[0], ge])) < 0):
        raise ValueError("group ends must be non-decreasing and end at M")


# ---- activations / gradients [M, C] -------------------------------------

def quantize_act(x_bf16, recipe: str, fmt: Fp8Format, group_ends=None,
                 rowwise: bool = True, colwise: bool = False,
                 dl_scale: Optional[tuple] = None, tensor_amax=None) -> dict:
    """Quantize a token-major tensor [M, C] (C = the feature dimension).

    Returns a dict with ``amax`` (tw/dl/nvfp4), ``row_codes`` [M, C] u8 and
    ``row_scales``; with colwise also ``padded_starts`` [E+1],
    ``col_codes`` [C, P_E] u8 and ``col_scales``. Scale layouts:
    tw/dl: float32 [1]; block: rows [M, C/128], cols [C, P_E/128];
    mx: uint8 E8M0 rows [M, C/32], cols [C, P_E/32]; nvfp4 (e2m1 codes):
    uint8 e4m3 block codes rows [M, C/16], cols [C, P_E/16], plus
    ``tensor_scale`` float32 [1].
    dl_scale = (s, inv) float32 from the delayed-scaling state.
    tensor_amax (nvfp4): the tensor unit's amax when x is a sample of a
    larger tensor (the tensor scale is that of the whole tensor).
    """
    x_bf16 = np.asarray(x_bf16, dtype=np.uint16)
    M, C = x_bf16.shape
    blk = {"block": BLOCK, "mx": MX_BLOCK}.get(recipe, BLOCK)
    if recipe not in RECIPES:
        raise ValueError(recipe)
    if C % BLOCK != 0:
        raise ValueError("feature dim must be a multiple of 128")
    x = bf16_to_f32(x_bf16)
    if recipe == "nvfp4":
        return _nvfp4_act(x, group_ends, rowwise, colwise, tensor_amax)
    out = {}
    if recipe in ("tw", "dl"):
        am = amax_of(x)
        out["amax"] = np.array([am], np.float32)
        if recipe == "tw":
            s, inv = fp32_scale_pair(am, fmt)
        else:
            s, inv = np.float32(dl_scale[0]), np.float32(dl_scale[1])
        s = np.float32(s)
        inv = np.float32(inv)
        if rowwise:
            out["row_codes"] = cast(x, inv, fmt)
            out["row_scales"] = np.array([s], np.float32)
        if colwise:
            check_groups(group_ends, M)
            P = padded_starts(group_ends)
            st = group_starts(group_ends)
            cc = np.zeros((C, int(P[-1])), np.uint8)
            for g in range(len(P) - 1):
                m = int(np.asarray(group_ends)[g] - st[g])
                # column-wise codes of a tensorwise unit are the row codes, moved
                cc[:, P[g]:P[g] + m] = cast(x[st[g]:st[g] + m, :], inv, fmt).T
            out["padded_starts"] = P
            out["col_codes"] = cc
            out["col_scales"] = np.array([s], np.float32)
        return out

    # blockwise (1x128 / 128x1) and MX (1x32 / 32x1)
    if rowwise:
        xb = x.reshape(M, C // blk, blk)
        am = np.max(np.abs(xb), axis=2) if M else np.zeros((0, C // blk), np.float32)
        codes, scales = _block_codes(xb, am, recipe, fmt)
        out["row_codes"] = codes.reshape(M, C)
        out["row_scales"] = scales
    if colwise:
        check_groups(group_ends, M)
        P = padded_starts(group_ends)
        st = group_starts(group_ends)
        Rp = int(P[-1])
        cc = np.zeros((C, Rp), np.uint8)
        if recipe == "block":
            cs = np.ones((C, Rp // blk), np.float32)
        else:
            cs = np.full((C, Rp // blk), E8M0_BIAS, np.uint8)
        ge = np.asarray(group_ends, dtype=np.int64)
        for g in range(len(P) - 1):
            m = int(ge[g] - st[g])
            for j0 in range(0, m, blk):        # units restart at the group's first row
                rows = x[st[g] + j0: st[g] + min(m, j0 + blk), :]      # [n<=blk, C]
                a = np.max(np.abs(rows), axis=0)                       # per feature column
                if recipe == "block":
                    s, inv = fp32_scale_pair(a, fmt)
                    cs[:, (P[g] + j0) // blk] = s
                else:
                    sc = mx_scale_codes(a, fmt)
                    inv = mx_inv_from_codes(sc)
                    cs[:, (P[g] + j0) // blk] = sc
                q = cast(rows, inv[None, :], fmt)                      # zero fill: the rest stays 0x00
                cc[:, P[g] + j0: P[g] + j0 + rows.shape[0]] = q.T
        out["padded_starts"] = P
        out["col_codes"] = cc
        out["col_scales"] = cs
    return out


def gather_rows(x_bf16, row_index) -> np.ndarray:
    """Routed rows A [M, C] of a token tensor x [T, C]: A[i] = x[row_index[i]].

    The grouped matmul is overridden for the routed experts only (torchao
    float8 MoE training PR, Limitations), whose operand holds each token's
    copies in expert order (the group offsets make every expert's rows one
    contiguous run). The permutation that builds it is a plain row gather;
    indices must lie in [0, T)."""
    x_bf16 = np.asarray(x_bf16, dtype=np.uint16)
    idx = np.asarray(row_index, dtype=np.int64)
    if idx.ndim != 1 or (idx.size and (idx.min() < 0 or idx.max() >= x_bf16.shape[0])):
        raise ValueError("row_index must be 1-D with entries in [0, T)")
    return x_bf16[idx]


def quantize_act_gather(x_bf16, row_index, recipe: str, fmt: Fp8Format, group_ends=None,
                        rowwise: bool = True, colwise: bool = False,
                        dl_scale: Optional[tuple] = None) -> dict:
    """``quantize_act`` of the routed rows ``gather_rows(x, row_index)``: the
    gather happens first, so every unit (including the tensorwise amax)
    covers the routed rows only."""
    return quantize_act(gather_rows(x_bf16, row_index), recipe, fmt, group_ends,
                        rowwise=rowwise, colwise=colwise, dl_scale=dl_scale)


def _block_codes(xb, am, recipe, fmt):
    """Codes and scales of blocks along the last axis; xb [..., nb, blk], am [..., nb]."""
    if recipe == "block":
        s, inv = fp32_scale_pair(am, fmt)
        return cast(xb, inv[..., None], fmt), s
    sc = mx_scale_codes(am, fmt)
    inv = mx_inv_from_codes(sc)
    return cast(xb, inv[..., None], fmt), sc


# ---- weights [E, K, N] ----------------------------------------------------

def quantize_weight(w_bf16, recipe: str, fmt: Fp8Format, dl_scale=None, tensor_amax=None) -> dict:
    """Quantize expert weights [E, K, N] (K contracts in forward, N in dgrad).

    Returns ``kmajor_codes`` [E, N, K] (forward operand, contiguous along K),
    ``nmajor_codes`` [E, K, N] (dgrad operand, contiguous along N) and their
    scales: tw/dl: float32 [E] for both (and ``amax`` [E]); block: 128x128
    tiles, float32 [E, K/128, N/128] for both (one code set, two layouts);
    mx: two code sets, ``kmajor_scales`` [E, N, K/32] (blocks along K) and
    ``nmajor_scales`` [E, K, N/32] (blocks along N); nvfp4: two e2m1 code
    sets with e4m3 block codes [E, N, K/16] and [E, K, N/16] and
    ``tensor_scale`` float32 [E] (one per expert, shared by both).
    dl_scale = (s[E], inv[E]) from the delayed-scaling state.
    """
    w_bf16 = np.asarray(w_bf16, dtype=np.uint16)
    E, K, N = w_bf16.shape
    if K % BLOCK or N % BLOCK:
        raise ValueError("K and N must be multiples of 128")
    w = bf16_to_f32(w_bf16)
    if recipe == "nvfp4":
        return _nvfp4_weight(w, tensor_amax)
    out = {}
    if recipe in ("tw", "dl"):
        am = np.array([amax_of(w[e]) for e in range(E)], np.float32)
        out["amax"] = am
        if recipe == "tw":
            s, inv = fp32_scale_pair(am, fmt)
        else:
            s = np.asarray(dl_scale[0], np.float32).reshape(E)
            inv = np.asarray(dl_scale[1], np.float32).reshape(E)
        nm = cast(w, inv[:, None, None], fmt)
        out["nmajor_codes"] = nm
        out["kmajor_codes"] = np.ascontiguousarray(nm.transpose(0, 2, 1))
        out["nmajor_scales"] = s.astype(np.float32)
        out["kmajor_scales"] = s.astype(np.float32)
        return out
    if recipe == "block":
        t = w.reshape(E, K // BLOCK, BLOCK, N // BLOCK, BLOCK)
        am = np.max(np.abs(t), axis=(2, 4))                          # [E, K/128, N/128]
        s, inv = fp32_scale_pair(am, fmt)
        nm = cast(t, inv[:, :, None, :, None], fmt).reshape(E, K, N)
        out["nmajor_codes"] = nm
        out["kmajor_codes"] = np.ascontiguousarray(nm.transpose(0, 2, 1))
        out["nmajor_scales"] = s
        out["kmajor_scales"] = s
        return out
    if recipe == "mx":
        # dgrad operand: blocks of 32 consecutive n in one row k
        tn = w.reshape(E, K, N // MX_BLOCK, MX_BLOCK)
        cn, sn = _block_codes(tn, np.max(np.abs(tn), axis=3), "mx", fmt)
        # forward operand: blocks of 32 consecutive k in one column n
        wt = np.ascontiguousarray(w.transpose(0, 2, 1))              # [E, N, K]
        tk = wt.reshape(E, N, K // MX_BLOCK, MX_BLOCK)
        ck, sk = _block_codes(tk, np.max(np.abs(tk), axis=3), "mx", fmt)
        out["nmajor_codes"] = cn.reshape(E, K, N)
        out["nmajor_scales"] = sn
        out["kmajor_codes"] = ck.reshape(E, N, K)
        out["kmajor_scales"] = sk
        return out
    raise ValueError(recipe)
