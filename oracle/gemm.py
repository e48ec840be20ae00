"""Grouped GEMM oracle in float64 on dequantized operands.

What is computed (the problem statement of the pages): per-expert token
groups [o_{g-1}, o_g) of a routed-row matrix, each multiplied by its own
expert's weight - the ``grouped_mm`` that the torchao float8 MoE PR
replaces by run-time quantization and a scaled grouped matmul (Summary), the
TEGroupedMLP / ``--moe-grouped-gemm`` path of the Megatron-LM bug report,
and equivalently the per-expert loop of SequentialMLP that report runs.
The backward (input gradients and parameter gradients) is the one the
torchao PR's test validates (Testing).

With deq(X)[i, j] = value(code[i, j]) * scale(unit of (i, j)) in float64:

* forward  Y[r, n]     = sum_k deq(A)[r, k]  * deq(W_g)[k, n],  r in group g
* dgrad    dA[r, k]    = sum_n deq(dY)[r, n] * deq(W_g)[k, n],  r in group g
* wgrad    dW_g[k, n]  = sum_{r in g} deq(A)[r, k] * deq(dY)[r, n]
  (an empty group gives 0, or leaves dW_g unchanged when accumulating)

Forward and dgrad outputs are bf16, wgrad is float32 (the main_grad
buffer of gradient-accumulation fusion in the single-grouped-weight PR's
table is float32); the oracle rounds its float64 result to the output
type (nearest, ties to even) before comparing.

Test infrastructure; see the package docstring.
"""
from __future__ import annotations

import numpy as np

from .formats import Fp8Format, E4M3, decode, e8m0_value
from .quant import BLOCK, MX_BLOCK, NV_BLOCK, group_starts


# ---- dequantization --------------------------------------------------------

def _expand(scales, rows: int, cols: int, blk: int) -> np.ndarray:
    """Broadcast per-(row, block) scales [rows, cols/blk] to [rows, cols]."""
    return np.repeat(np.asarray(scales, np.float64), blk, axis=1)[:rows, :cols]


def deq_act_rows(codes, scales, recipe: str, fmt: Fp8Format) -> np.ndarray:
    """float64 [M, C] of a row-wise quantized token tensor. For nvfp4,
    ``scales`` is (e4m3 block codes [M, C/16], tensor scale)."""
    v = decode(codes, fmt)
    M, C = v.shape
    if recipe == "nvfp4":
        blocks, s_t = scales
        return v * _expand(decode(blocks, E4M3), M, C, NV_BLOCK) * float(np.asarray(s_t).reshape(-1)[0])
    if recipe in ("tw", "dl"):
        return v * float(np.asarray(scales).reshape(-1)[0])
    if recipe == "block":
        return v * _expand(scales, M, C, BLOCK)
    return v * _expand(e8m0_value(scales), M, C, MX_BLOCK)


def deq_act_cols(codes, scales, recipe: str, fmt: Fp8Format) -> np.ndarray:
    """float64 [C, Rp] of a column-wise (transposed, padded) token tensor."""
    return deq_act_rows(codes, scales, recipe, fmt)


def deq_weight(q: dict, recipe: str, fmt: Fp8Format, layout: str) -> np.ndarray:
    """float64 [E, K, N] of a quantized weight, from its k-major or n-major codes.

    layout "k": the forward operand (codes [E, N, K]); "n": the dgrad
    operand (codes [E, K, N]). Both give W in [E, K, N] orientation.
    """
    if layout == "k":
        codes = np.asarray(q["kmajor_codes"])           # [E, N, K]
        scales = q["kmajor_scales"]
    else:
        codes = np.asarray(q["nmajor_codes"])           # [E, K, N]
        scales = q["nmajor_scales"]
    v = decode(codes, fmt)
    E = v.shape[0]
    if recipe == "nvfp4":
        s_t = np.asarray(q["tensor_scale"], np.float64).reshape(E, 1, 1)
        d = v * np.repeat(decode(scales, E4M3), NV_BLOCK, axis=2) * s_t
    elif recipe in ("tw", "dl"):
        d = v * np.asarray(scales, np.float64).reshape(E, 1, 1)
    elif recipe == "block":
        s = np.asarray(scales, np.float64)              # [E, K/128, N/128]
        s_full = np.repeat(np.repeat(s, BLOCK, axis=1), BLOCK, axis=2)   # [E, K, N]
        d = v * (s_full.transpose(0, 2, 1) if layout == "k" else s_full)
    else:
        sv = e8m0_value(scales)                         # [E, rows, cols/32] along the code rows
        d = v * np.repeat(sv, MX_BLOCK, axis=2)
    return d.transpose(0, 2, 1) if layout == "k" else d


# ---- grouped GEMM (float64) -------------------------------------------------

def grouped_fwd(A, W, group_ends) -> np.ndarray:
    """Y [M, N] = A_g @ W_g for each group (float64)."""
    A = np.asarray(A, np.float64)
    W = np.asarray(W, np.float64)
    st = group_starts(group_ends)
    Y = np.zeros((A.shape[0], W.shape[2]), np.float64)
    for g, (a, b) in enumerate(zip(st, np.asarray(group_ends, np.int64))):
        if b > a:
            Y[a:b] = A[a:b] @ W[g]
    return Y


def grouped_dgrad(dY, W, group_ends) -> np.ndarray:
    """dA [M, K] = dY_g @ W_g^T for each group (float64)."""
    dY = np.asarray(dY, np.float64)
    W = np.asarray(W, np.float64)
    st = group_starts(group_ends)
    dA = np.zeros((dY.shape[0], W.shape[1]), np.float64)
    for g, (a, b) in enumerate(zip(st, np.asarray(group_ends, np.int64))):
        if b > a:
            dA[a:b] = dY[a:b] @ W[g].T
    return dA


def grouped_wgrad(A, dY, group_ends, E: int, init=None) -> np.ndarray:
    """dW [E, K, N] = A_g^T @ dY_g (float64); init (if given) is added."""
    A = np.asarray(A, np.float64)
    dY = np.asarray(dY, np.float64)
    st = group_starts(group_ends)
    dW = np.zeros((E, A.shape[1], dY.shape[1]), np.float64)
    if init is not None:
        dW += np.asarray(init, np.float64)
    for g, (a, b) in enumerate(zip(st, np.asarray(group_ends, np.int64))):
        if b > a:
            dW[g] += A[a:b].T @ dY[a:b]
    return dW


def unpad_cols(col_deq, padded_starts, group_ends) -> np.ndarray:
    """Token-major [M, C] from a column-wise padded [C, Rp] operand."""
    st = group_starts(group_ends)
    ge = np.asarray(group_ends, np.int64)
    C = col_deq.shape[0]
    out = np.zeros((int(ge[-1]) if ge.size else 0, C), np.float64)
    for g in range(len(ge)):
        m = int(ge[g] - st[g])
        out[st[g]:st[g] + m] = col_deq[:, padded_starts[g]:padded_starts[g] + m].T
    return out


# ---- output rounding and error measures ------------------------------------

def round_bf16(x) -> np.ndarray:
    """float64 -> nearest bf16 value (ties to even), returned as float64.

    Done directly from float64 (no float32 step, so no double rounding):
    the significand is rounded to 8 bits; below 2^-126 the quantum is 2^-133.
    """
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)                       # x = m * 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                  # subnormal range: fixed quantum 2^-133
    q = np.rint(np.ldexp(m, 8 + (np.frexp(x)[1] - e)))   # significand in units of 2^(e-8)
    y = np.ldexp(q, e - 8)
    y = np.where(np.abs(y) >= 2.0 ** 128, np.copysign(np.inf, x), y)
    return np.where(x == 0, x, y)


def round_f32(x) -> np.ndarray:
    return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)


def bf16_bits_to_f64(b) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def rel_fro(y, ref) -> float:
    """||y - ref||_F / ||ref||_F (0 when both are zero)."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(y - ref)
    if den == 0:
        return 0.0 if num == 0 else float("inf")
    return float(num / den)


def sqnr_db(ref, y) -> float:
    """10 log10(||ref||^2 / ||ref - y||^2)."""
    ref = np.asarray(ref, np.float64)
    err = np.linalg.norm(ref - np.asarray(y, np.float64))
    if err == 0:
        return float("inf")
    return float(20.0 * np.log10(np.linalg.norm(ref) / err))
