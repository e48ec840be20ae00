"""Seeded synthetic inputs for the five expert-GEMM workloads.

This module only draws random numbers and lays them out: token routing,
bf16 activations / weights / output gradients and the per-expert group
ends. It holds none of the quantization or GEMM arithmetic, so both the
CPU oracle (through the tests) and the HIP path can be fed from it.

Every tensor is drawn with ``numpy.random.default_rng(SeedSequence([cid,
tensor_id, step]))`` as float32, then rounded to bf16 (round to nearest
even) and returned as uint16 bit patterns, the exact bits both sides see.
Routing is drawn as each token's top-k expert choices; grouping the routed
rows by expert is a step of the path (the device kernel, checked against
the oracle), not done here.

Workload shapes follow the problem statement of the float8 MoE training
pages: a tiny four-expert case, a Mixtral-8x7B-shaped expert FFN (the
Megatron-LM FP8-vs-BF16 bug report trains Mixtral 8x7B), the same shape
with delayed scaling and hybrid formats (that report's
``--fp8-format hybrid --fp8-amax-history-len 1024`` run), a DeepSeek-style
blockwise case (the Transformer Engine Float8BlockQuantizer issue) and a
Llama4-Scout-shaped MXFP8 case (the torchao float8 MoE prototype tests a
Llama4 MoE layer; the Megatron single-grouped-weight PR tests MXFP8).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

# tensor ids used in the seed sequence
T_X, T_LOGITS, T_W1, T_W2, T_A2, T_DY1, T_DY2, T_OUTLIER, T_ROUTE = range(9)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); return uint16 bits.

    Inputs here are finite, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(cid: int, tid: int, step: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cid, tid, step]))


def normal_bf16(cid: int, tid: int, shape, std: float = 1.0, step: int = 0,
                chunk_rows: int = 1 << 12) -> np.ndarray:
    """bf16 bits of N(0, std^2) draws of the given shape, drawn in row chunks."""
    shape = tuple(int(s) for s in shape)
    rng = _rng(cid, tid, step)
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(-1, shape[-1])
    std32 = np.float32(std)
    for r0 in range(0, flat.shape[0], chunk_rows):
        r1 = min(flat.shape[0], r0 + chunk_rows)
        v = rng.standard_normal((r1 - r0, shape[-1]), dtype=np.float32)
        if std != 1.0:
            v *= std32
        flat[r0:r1] = bf16_bits(v)
    return out


@dataclasses.dataclass
class TopK:
    """Top-k expert choices of every token (the router's output, before the
    routed rows are grouped by expert)."""
    n_tokens: int
    n_experts: int
    expert_ids: np.ndarray   # int32 [T, k], in choice order

    @property
    def k(self) -> int:
        return int(self.expert_ids.shape[1])

    @property
    def rows(self) -> int:
        return self.n_tokens * self.k


def route_topk(cid: int, n_tokens: int, n_experts: int, k: int,
               masked=(), uniform: bool = False) -> TopK:
    """Top-k routing. uniform: k distinct experts uniformly at random;
    otherwise the k largest of N(0,1) logits (softmax does not change the
    order), with ``masked`` experts never chosen. Ties go to the lower id.
    Choices are listed by descending key."""
    rng = _rng(cid, T_LOGITS)
    if uniform:
        keys = rng.random((n_tokens, n_experts))
    else:
        keys = rng.standard_normal((n_tokens, n_experts), dtype=np.float32).astype(np.float64)
    for e in masked:
        keys[:, e] = -np.inf
    # descending by key, ascending by expert id on ties
    order = np.lexsort((np.broadcast_to(np.arange(n_experts), keys.shape), -keys), axis=1)
    return TopK(n_tokens, n_experts, np.ascontiguousarray(order[:, :k]).astype(np.int32))


def route_zipf(cid: int, n_tokens: int, n_experts: int, alpha: float) -> TopK:
    """Top-1 routing with P(e) proportional to (e+1)^-alpha."""
    rng = _rng(cid, T_ROUTE)
    p = (np.arange(1, n_experts + 1, dtype=np.float64)) ** (-alpha)
    p /= p.sum()
    exp = rng.choice(n_experts, size=n_tokens, p=p)
    return TopK(n_tokens, n_experts, exp.reshape(-1, 1).astype(np.int32))


def group_ends_from_sizes(sizes) -> np.ndarray:
    return np.cumsum(np.asarray(sizes, dtype=np.int64)).astype(np.int32)


@dataclasses.dataclass(frozen=True)
class WorkloadSpec:
    cid: int
    name: str
    experts: int
    tokens: int
    topk: int
    hidden: int            # K of the gate/up GEMM
    ffn: int               # per-expert FFN width
    recipe: str            # "tw", "dl", "block", "mx", "mxfp4" (MX with e2m1 elements), "nvfp4"
    modes: tuple           # subset of ("fwd", "dgrad", "wgrad")
    gemms: tuple           # ("gu",) or ("gu", "dn")
    steps: int = 1

    @property
    def gu_n(self) -> int:
        # tiny case: up-projection only, N = ffn; otherwise gate+up fused, N = 2*ffn
        return self.ffn if self.gemms == ("gu",) else 2 * self.ffn

    def gemm_shape(self, which: str):
        """(K, N) of the named expert GEMM."""
        return (self.hidden, self.gu_n) if which == "gu" else (self.ffn, self.hidden)


SPECS: Dict[int, WorkloadSpec] = {
    1: WorkloadSpec(1, "tiny-moe-e4-h256-f512-tw", 4, 512, 2, 256, 512, "tw",
                    ("fwd",), ("gu",)),
    2: WorkloadSpec(2, "mixtral-8x7b-experts-tw", 8, 8192, 2, 4096, 14336, "tw",
                    ("fwd",), ("gu", "dn")),
    3: WorkloadSpec(3, "mixtral-8x7b-experts-delayed-hybrid", 8, 8192, 2, 4096, 14336, "dl",
                    ("fwd", "dgrad", "wgrad"), ("gu", "dn"), steps=50),
    4: WorkloadSpec(4, "deepseek-style-e64-blockwise", 64, 16384, 6, 2048, 1408, "block",
                    ("fwd", "dgrad", "wgrad"), ("gu", "dn")),
    5: WorkloadSpec(5, "llama4-scout-experts-mxfp8", 16, 16384, 1, 5120, 8192, "mx",
                    ("fwd", "dgrad", "wgrad"), ("gu", "dn")),
    # the MXFP4 variant of the same shapes: e2m1 elements for every operand
    6: WorkloadSpec(6, "llama4-scout-experts-mxfp4", 16, 16384, 1, 5120, 8192, "mxfp4",
                    ("fwd", "dgrad", "wgrad"), ("gu", "dn")),
    # the NVFP4 variant: e2m1 elements, e4m3 scale per 16, fp32 per tensor
    7: WorkloadSpec(7, "llama4-scout-experts-nvfp4", 16, 16384, 1, 5120, 8192, "nvfp4",
                    ("fwd", "dgrad", "wgrad"), ("gu", "dn")),
}

C4_MASKED = (0, 21, 42, 63)


def routing_for(cid: int) -> TopK:
    """The workload's top-k expert choices."""
    s = SPECS[cid]
    if cid == 1:
        return route_topk(cid, s.tokens, s.experts, s.topk, uniform=True)
    if cid in (2, 3):
        return route_topk(2, s.tokens, s.experts, s.topk)   # C3 reuses C2's routing
    if cid == 4:
        return route_topk(cid, s.tokens, s.experts, s.topk, masked=C4_MASKED)
    if cid in (5, 6, 7):
        return route_zipf(5, s.tokens, s.experts, 1.1)   # the FP4 variants reuse C5's routing
    raise KeyError(cid)


def token_activation(cid: int, step: int = 0) -> np.ndarray:
    """Token rows x [tokens, hidden] of the gate/up GEMM input (before the
    routed rows are gathered). C3 scales by 1.01**step (drift), C5/C6
    multiply 0.1% of elements by 50."""
    s = SPECS[cid]
    std = 1.01 ** step if cid == 3 else 1.0
    x = normal_bf16(cid, T_X, (s.tokens, s.hidden), std=std, step=step)
    if cid in (5, 6, 7):
        x = _outliers(cid, T_X, x)
    return x


def down_activation(cid: int, rows: int, step: int = 0) -> np.ndarray:
    """Routed-row input of the down GEMM [rows, ffn], drawn per row (same
    drift and outliers as the token rows)."""
    s = SPECS[cid]
    std = 1.01 ** step if cid == 3 else 1.0
    a = normal_bf16(cid, T_A2, (rows, s.ffn), std=std, step=step)
    if cid in (5, 6, 7):
        a = _outliers(cid, T_A2, a)
    return a


def _outliers(cid: int, tid: int, x: np.ndarray) -> np.ndarray:
    """Multiply 0.1% of elements (seeded, without replacement) by 50."""
    rng = _rng(cid, T_OUTLIER * 16 + tid)
    n = x.size
    idx = rng.choice(n, size=max(1, n // 1000), replace=False)
    flat = x.reshape(-1)
    v = bf16_to_f32(flat[idx]) * np.float32(50.0)
    flat[idx] = bf16_bits(v)
    return x


def weight_bf16(cid: int, which: str) -> np.ndarray:
    """Expert weights [E, K, N] ~ N(0, 0.02^2)."""
    s = SPECS[cid]
    K, N = s.gemm_shape(which)
    return normal_bf16(cid, T_W1 if which == "gu" else T_W2, (s.experts, K, N), std=0.02)


def grad_bf16(cid: int, which: str, rows: int, step: int = 0) -> np.ndarray:
    """Output gradient dY [rows, N] = N(0,1) * 2^-10 (a power of two keeps scale equivariance)."""
    s = SPECS[cid]
    N = s.gemm_shape(which)[1]
    return normal_bf16(cid, T_DY1 if which == "gu" else T_DY2, (rows, N),
                       std=2.0 ** -10, step=step)


def small_case(seed: int, sizes: List[int], K: int, N: int, w_std: float = 0.02,
               outlier: bool = False):
    """A small ragged case for parity tests: returns (A [R,K], W [E,K,N], dY [R,N], group_ends)."""
    E = len(sizes)
    R = int(sum(sizes))
    a = normal_bf16(1000 + seed, T_X, (max(R, 1), K))[:R]
    if outlier and R:
        a = _outliers(1000 + seed, T_X, a)
    w = normal_bf16(1000 + seed, T_W1, (E, K, N), std=w_std)
    dy = normal_bf16(1000 + seed, T_DY1, (max(R, 1), N), std=2.0 ** -10)[:R]
    return a, w, dy, group_ends_from_sizes(sizes)
