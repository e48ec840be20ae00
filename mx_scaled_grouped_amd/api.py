"""Torch-facing binding of the C ABI in include/mxsg.h.

PyTorch supplies device memory and the current HIP stream; every step of
the computation runs in the HIP kernels of libmxsg.so. Functions here
only allocate outputs, check dtypes / devices and pass pointers.

The calls follow the problem statement of the float8 MoE pages:
``quantize(tensor, recipe)`` for routed-row activations, gradients and
expert weights, and ``grouped_mm`` for the forward, dgrad and wgrad
products over per-expert token groups.
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import List, Optional

import torch

from . import _lib

E4M3, E5M2, E2M1 = 0, 1, 2
FMT = {"e4m3": E4M3, "e5m2": E5M2, "e2m1": E2M1, E4M3: E4M3, E5M2: E5M2, E2M1: E2M1}


def elems_per_byte(fmt) -> int:
    """Elements per code byte: 2 for 4-bit e2m1 (MXFP4), else 1."""
    return 2 if FMT[fmt] == E2M1 else 1
RECIPES = {"tw": 0, "dl": 1, "block": 2, "mx": 3, "nvfp4": 4}
MODE_FWD, MODE_DGRAD, MODE_WGRAD = 0, 1, 2


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _check_dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("tensors must be on the GPU")
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _need(t: Optional[torch.Tensor], nbytes: int, what: str, dtype=None) -> None:
    """The C ABI takes bare pointers, so the binding checks every buffer it
    passes: a buffer smaller than the call writes or reads would be an
    out-of-bounds access on the device."""
    if t is None:
        raise ValueError(f"{what} is missing")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype}, got {t.dtype}")
    if _nbytes(t) < nbytes:
        raise ValueError(f"{what} holds {_nbytes(t)} bytes, the call needs {nbytes}")


def _bits16(x: torch.Tensor) -> torch.Tensor:
    if x.dtype == torch.bfloat16:
        return x
    if x.dtype in (torch.int16, torch.uint16):
        return x
    raise TypeError("expected bf16 (or its 16-bit bit pattern)")


def padded_capacity(M: int, E: int) -> int:
    """Columns of the column-wise layout for M tokens in E groups."""
    return int(_lib.load().mxsg_padded_capacity(M, E))


def unpack_codes(t: torch.Tensor, rows: Optional[int] = None) -> torch.Tensor:
    """Row-major copy [..., rows, L] of pair-interleaved codes [..., Rp, L].

    The library stores every code matrix pair-interleaved: rows 2p and 2p+1
    share 2L bytes as 128-byte lines, each 64 bytes of row 2p followed by the
    same 64 bytes of row 2p+1 (mxsg.h, Layouts)."""
    *lead, rp, L = t.shape
    if rp % 2 or L % 64:
        raise ValueError(f"pair-interleaved codes need an even row count and L % 64 == 0, got {tuple(t.shape)}")
    u = t.reshape(*lead, rp // 2, L // 64, 2, 64).transpose(-3, -2).reshape(*lead, rp, L)
    return u if rows is None else u[..., :rows, :]


def pack_codes(t: torch.Tensor) -> torch.Tensor:
    """Pair-interleaved copy of row-major codes [..., R, L] (R rounded up to
    even with a zero row)."""
    *lead, r, L = t.shape
    if L % 64:
        raise ValueError(f"row length {L} is not a multiple of 64")
    if r % 2:
        t = torch.cat([t, t.new_zeros(*lead, 1, L)], dim=-2)
        r += 1
    return t.reshape(*lead, r // 2, 2, L // 64, 64).transpose(-3, -2).reshape(*lead, r, L).contiguous()


def unpack_mx_scales(t: torch.Tensor) -> torch.Tensor:
    """Row-major copy [..., R, 4W] of word-major E8M0 scales [..., W, R, 4].

    The library stores MX scale matrices word-major: word w (the four
    32-blocks of contraction elements [128w, 128w + 128)) of every row,
    rows consecutive, then word w + 1 (mxsg.h, Layouts)."""
    *lead, w, r, four = t.shape
    if four != 4:
        raise ValueError(f"word-major scales need a last dimension of 4, got {tuple(t.shape)}")
    return t.transpose(-3, -2).reshape(*lead, r, 4 * w)


def pack_mx_scales(t: torch.Tensor) -> torch.Tensor:
    """Word-major copy [..., B/4, R, 4] of row-major E8M0 scales [..., R, B]."""
    *lead, r, b = t.shape
    if b % 4:
        raise ValueError(f"block count {b} is not a multiple of 4")
    return t.reshape(*lead, r, b // 4, 4).transpose(-3, -2).contiguous()


# status word bits (mxsg.h)
STATUS_ENDS_DECREASING, STATUS_ENDS_RANGE, STATUS_ENDS_TOTAL, STATUS_NONFINITE = 1, 2, 4, 8
STATUS_BAD_EXPERT = 16


def _status_word(t: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if t is not None and (t.dtype != torch.int32 or t.numel() < 1):
        raise TypeError("status must be an int32 device tensor with at least one element")
    return t


def _scale_blocks(recipe: str) -> int:
    return {"block": 128, "mx": 32}.get(recipe, 0)


def _scale_dtype(recipe: str) -> torch.dtype:
    """E8M0 (MX) and e4m3 (NVFP4) scale codes are bytes; the rest fp32."""
    return torch.uint8 if recipe in ("mx", "nvfp4") else torch.float32


# NVFP4 code order inside each 128-element (64-byte) piece of a row: the 8
# elements 16 s + 8 h .. + 7 (k16 step s, half h) form the dword at byte
# 32 (s // 4) + 16 h + 4 (s % 4) (mxsg.h, Layouts).
def _nv_nibble_order() -> torch.Tensor:
    """nibble position of logical element e of a 128-element piece"""
    pos = []
    for e in range(128):
        st, h, i = e // 16, (e // 8) % 2, e % 8
        byte = 32 * (st // 4) + 16 * h + 4 * (st % 4) + i // 2
        pos.append(2 * byte + i % 2)
    return torch.tensor(pos, dtype=torch.long)


def unpack_nvfp4_codes(t: torch.Tensor, rows: Optional[int] = None) -> torch.Tensor:
    """Row-major e2m1 codes [..., rows, L], one per uint8, from NVFP4 code
    bytes [..., Rp, L/2] (pair-interleaved rows, NVFP4 nibble order)."""
    b = unpack_codes(t, rows)
    nib = torch.stack([b & 0xF, b >> 4], dim=-1).reshape(*b.shape[:-1], -1)       # nibbles in storage order
    L = nib.shape[-1]
    idx = _nv_nibble_order().to(nib.device)
    piece = nib.reshape(*nib.shape[:-1], L // 128, 128)
    return piece.index_select(-1, idx).reshape(*nib.shape[:-1], L)


def pack_nvfp4_codes(codes: torch.Tensor) -> torch.Tensor:
    """NVFP4 code bytes [..., R + R % 2, L/2] (pair-interleaved rows, NVFP4
    nibble order) from row-major e2m1 codes [..., R, L], one per uint8."""
    *lead, r, L = codes.shape
    if L % 128:
        raise ValueError(f"row length {L} is not a multiple of 128")
    pos = _nv_nibble_order().to(codes.device)
    piece = codes.reshape(*lead, r, L // 128, 128)
    stored = torch.empty_like(piece)
    stored[..., pos] = piece                                    # element e goes to nibble position pos[e]
    nib = stored.reshape(*lead, r, L // 2, 2)
    return pack_codes((nib[..., 0] | (nib[..., 1] << 4)).contiguous())


def pack_nvfp4_scales(blocks: torch.Tensor, tensor_scales: torch.Tensor) -> torch.Tensor:
    """An NVFP4 scale buffer (uint8) from e4m3 block codes [units, rows, L/16]
    and fp32 tensor scales [units]: each unit's codes piece-major
    [L/128, rows, 8], then the tensor scales."""
    units, rows, nb = blocks.shape
    pm = blocks.reshape(units, rows, nb // 8, 8).transpose(1, 2).reshape(-1)
    ts = tensor_scales.to(torch.float32).contiguous().view(torch.uint8)
    return torch.cat([pm.to(torch.uint8), ts.to(pm.device)])


def nvfp4_scales(t: torch.Tensor, rows: int, L: int, units: int = 1):
    """(e4m3 block codes [units, rows, L/16], tensor scales float32 [units])
    of an NVFP4 scale buffer: each unit's block codes piece-major
    ([L/128, rows, 8]), the units' codes one after another, then the fp32
    tensor scales."""
    flat = t.reshape(-1)
    n = rows * (L // 16)
    blocks = flat[:units * n].reshape(units, L // 128, rows, 8).transpose(1, 2).reshape(units, rows, L // 16)
    ts = flat[units * n:units * n + 4 * units].view(torch.float32)
    return blocks, ts


def quantize_act_sizes(M: int, C: int, recipe: str, fmt=E4M3, E: int = 0) -> List[int]:
    """Byte sizes [row_codes, row_scales, col_codes, col_scales,
    padded_starts] of mxsg_quantize_act's outputs (E = 0: row-wise only)."""
    out = (ctypes.c_int64 * 5)()
    _lib.call("mxsg_quantize_act_sizes", M, C, RECIPES[recipe], FMT[fmt], E, ctypes.addressof(out))
    return list(out)


def quantize_weight_sizes(E: int, K: int, N: int, recipe: str, fmt=E4M3) -> List[int]:
    """Byte sizes [kmajor_codes, kmajor_scales, nmajor_codes, nmajor_scales]
    of mxsg_quantize_weight's outputs."""
    out = (ctypes.c_int64 * 4)()
    _lib.call("mxsg_quantize_weight_sizes", E, K, N, RECIPES[recipe], FMT[fmt], ctypes.addressof(out))
    return list(out)


def _buffer(nbytes: int, dtype: torch.dtype, cols: int, dev) -> torch.Tensor:
    """A [nbytes / itemsize / cols, cols] tensor (cols = 0: a flat one)."""
    n = nbytes // torch.empty(0, dtype=dtype).element_size()
    t = torch.empty(n, dtype=dtype, device=dev)
    return t.view(-1, cols) if cols else t


@dataclasses.dataclass
class Route:
    """Device routing of top-k choices (mxsg_route)."""
    group_ends: torch.Tensor                 # int32 [E]
    row_index: torch.Tensor                  # int32 [T * k]: routed row -> token
    slot_row: Optional[torch.Tensor] = None  # int32 [T * k]: choice -> routed row


def route(expert_ids: torch.Tensor, E: int, slot_row: bool = False, out: Optional[Route] = None,
          status: Optional[torch.Tensor] = None) -> Route:
    """Group the routed rows by expert on the device (mxsg_route).
    ``expert_ids`` is int32 [T, k]; rows are ordered by expert, then token,
    then choice. ``out`` reuses a previous Route's buffers."""
    _check_dev(expert_ids, status)
    if expert_ids.dtype != torch.int32 or expert_ids.dim() != 2:
        raise TypeError("expert_ids must be a 2-D int32 tensor [T, k]")
    T, k = expert_ids.shape
    dev = expert_ids.device
    if out is None:
        out = Route(torch.empty(E, dtype=torch.int32, device=dev),
                    torch.empty(T * k, dtype=torch.int32, device=dev),
                    torch.empty(T * k, dtype=torch.int32, device=dev) if slot_row else None)
    _check_dev(out.group_ends, out.row_index, out.slot_row)
    _need(out.group_ends, 4 * E, "out.group_ends", torch.int32)
    _need(out.row_index, 4 * T * k, "out.row_index", torch.int32)
    if slot_row:
        _need(out.slot_row, 4 * T * k, "out.slot_row", torch.int32)
    _lib.call("mxsg_route", _ptr(expert_ids), T, k, E, _ptr(out.group_ends), _ptr(out.row_index),
              _ptr(out.slot_row) if slot_row else None, _ptr(_status_word(status)), _stream())
    return out


@dataclasses.dataclass
class DelayedState:
    """Caller-owned delayed-scaling state for `units` scaling units of one format."""
    history: torch.Tensor   # fp32 [units, L]
    pos: torch.Tensor       # int32 [units]
    amax: torch.Tensor      # fp32 [units]
    scale: torch.Tensor     # fp32 [units]
    inv: torch.Tensor       # fp32 [units]
    fmt: int

    @classmethod
    def create(cls, units: int, fmt, history_len: int = 1024, device="cuda") -> "DelayedState":
        f = torch.float32
        return cls(torch.zeros(units, history_len, dtype=f, device=device),
                   torch.zeros(units, dtype=torch.int32, device=device),
                   torch.zeros(units, dtype=f, device=device),
                   torch.ones(units, dtype=f, device=device),
                   torch.ones(units, dtype=f, device=device), FMT[fmt])

    @property
    def units(self) -> int:
        return self.history.shape[0]

    def update(self) -> None:
        """Push each unit's recorded amax and recompute its scale (mxsg_delayed_update)."""
        _lib.call("mxsg_delayed_update", _ptr(self.history), _ptr(self.pos), _ptr(self.amax),
                  _ptr(self.scale), _ptr(self.inv), self.units, self.history.shape[1], self.fmt,
                  _stream())

    def state_dict(self):
        return {k: getattr(self, k).detach().cpu().clone() for k in ("history", "pos", "amax", "scale", "inv")}

    def load_state_dict(self, d):
        for k, v in d.items():
            getattr(self, k).copy_(v)


def _check_quant_act_out(q: "QuantAct", recipe: str, f: int, M: int, C: int, E: int,
                         rowwise: bool, colwise: bool) -> None:
    """A reused QuantAct must describe the same call: same recipe, format
    and shape, the requested layouts present, and every buffer at least the
    size mxsg_quantize_act_sizes gives."""
    if (q.recipe, q.fmt, q.M, q.C) != (recipe, f, M, C):
        raise ValueError(f"out was made for recipe={q.recipe} fmt={q.fmt} M={q.M} C={q.C}, "
                         f"the call has recipe={recipe} fmt={f} M={M} C={C}")
    nb = quantize_act_sizes(M, C, recipe, f, E if colwise else 0)
    sdt = _scale_dtype(recipe)
    if rowwise:
        _need(q.row_codes, nb[0], "out.row_codes", torch.uint8)
        _need(q.row_scales, nb[1], "out.row_scales", sdt)
    elif q.row_codes is not None:
        raise ValueError("out holds row-wise codes but the call asks for none")
    if colwise:
        if q.ld != padded_capacity(M, E):
            raise ValueError(f"out.ld={q.ld} was made for another group count (need {padded_capacity(M, E)})")
        _need(q.col_codes, nb[2], "out.col_codes", torch.uint8)
        _need(q.col_scales, nb[3], "out.col_scales", sdt)
        _need(q.padded_starts, nb[4], "out.padded_starts", torch.int32)
    elif q.col_codes is not None:
        raise ValueError("out holds column-wise codes but the call asks for none")
    if recipe in ("tw", "nvfp4"):
        _need(q.amax, 4, "out.amax", torch.float32)


@dataclasses.dataclass
class QuantAct:
    recipe: str
    fmt: int
    M: int
    C: int
    row_codes: Optional[torch.Tensor] = None     # uint8 [M + M % 2, C] (C/2 for e2m1), pair-interleaved
    row_scales: Optional[torch.Tensor] = None
    col_codes: Optional[torch.Tensor] = None     # uint8 [C, ld] (ld/2 for e2m1), pair-interleaved
    col_scales: Optional[torch.Tensor] = None
    padded_starts: Optional[torch.Tensor] = None  # int32 [E+1]
    amax: Optional[torch.Tensor] = None
    ld: int = 0


def quantize_act(x: torch.Tensor, recipe: str, fmt, group_ends: Optional[torch.Tensor] = None,
                 rowwise: bool = True, colwise: bool = False,
                 state: Optional[DelayedState] = None, unit: int = 0,
                 out: Optional[QuantAct] = None,
                 row_index: Optional[torch.Tensor] = None,
                 status: Optional[torch.Tensor] = None, swiglu: bool = False) -> QuantAct:
    """Quantize a token-major bf16 tensor [M, C] (mxsg_quantize_act).

    recipe "dl" takes its scale from ``state`` unit ``unit`` and records
    the amax there. Column-wise output needs ``group_ends`` (int32 [E]).
    ``out`` reuses previously allocated outputs of the same shape.
    With ``row_index`` (int32 [M]) the operand is the routed rows
    x[row_index] of a token tensor x [T, C], gathered inside the kernel
    (mxsg_quantize_act_gather). ``status`` (int32 [1], device) receives the
    MXSG_STATUS_* bits of malformed group ends and non-finite inputs.
    With ``swiglu`` x is a gate/up output [M, 2C] and the quantized tensor
    is its SwiGLU activation silu(gate) * up [M, C]
    (mxsg_quantize_act_swiglu; not with ``row_index``).
    """
    x = _bits16(x)
    _check_dev(x, group_ends, row_index, status)
    T, C = x.shape
    if swiglu:
        if row_index is not None:
            raise ValueError("swiglu takes routed rows in order (no row_index)")
        if C % 2:
            raise ValueError("a gate/up output has an even number of columns")
        C //= 2
    if row_index is not None:
        if row_index.dtype != torch.int32 or row_index.dim() != 1:
            raise TypeError("row_index must be a 1-D int32 tensor")
        M = int(row_index.numel())
    else:
        M = T
    f = FMT[fmt]
    dev = x.device
    blk = _scale_blocks(recipe)
    E = int(group_ends.numel()) if group_ends is not None else 0
    if colwise and group_ends is None:
        raise ValueError("column-wise output needs group_ends")
    if group_ends is not None and group_ends.dtype != torch.int32:
        raise TypeError("group_ends must be int32")
    q = out
    if q is not None:
        _check_quant_act_out(q, recipe, f, M, C, E, rowwise, colwise)
    else:
        q = QuantAct(recipe, f, M, C)
        sdt = _scale_dtype(recipe)
        nb = quantize_act_sizes(M, C, recipe, f, E if colwise else 0)
        epb = elems_per_byte(f)
        if rowwise:
            q.row_codes = _buffer(nb[0], torch.uint8, C // epb, dev)
            q.row_scales = _buffer(nb[1], sdt, C // blk if blk else 0, dev)
            if recipe == "mx":  # word-major [C/128, M, 4]
                q.row_scales = q.row_scales.view(C // 128, M, 4)
        if colwise:
            q.ld = padded_capacity(M, E)
            q.col_codes = _buffer(nb[2], torch.uint8, q.ld // epb, dev)
            q.col_scales = _buffer(nb[3], sdt, q.ld // blk if blk else 0, dev)
            if recipe == "mx":  # word-major [ld/128, C, 4]
                q.col_scales = q.col_scales.view(q.ld // 128, C, 4)
            q.padded_starts = _buffer(nb[4], torch.int32, 0, dev)
        if recipe in ("tw", "nvfp4"):
            q.amax = torch.empty(1, dtype=torch.float32, device=dev)
    amax = q.amax
    dls = dli = None
    if recipe == "dl":
        if state is None:
            raise ValueError("recipe 'dl' needs a DelayedState")
        if not 0 <= unit < state.units:
            raise ValueError(f"unit {unit} outside the state's {state.units} units")
        amax = state.amax[unit:unit + 1]
        dls = state.scale[unit:unit + 1]
        dli = state.inv[unit:unit + 1]
    outs = (E, _ptr(group_ends), _ptr(q.row_codes), _ptr(q.row_scales), _ptr(q.col_codes),
            _ptr(q.col_scales), q.ld, _ptr(q.padded_starts), _ptr(amax), _ptr(dls), _ptr(dli),
            _ptr(_status_word(status)), _stream())
    if swiglu:
        _lib.call("mxsg_quantize_act_swiglu", _ptr(x), M, C, RECIPES[recipe], f, *outs)
    elif row_index is None:
        _lib.call("mxsg_quantize_act", _ptr(x), M, C, RECIPES[recipe], f, *outs)
    else:
        _lib.call("mxsg_quantize_act_gather", _ptr(x), T, _ptr(row_index), M, C, RECIPES[recipe],
                  f, *outs)
    return q


def _check_quant_weight_out(q: "QuantWeight", recipe: str, f: int, E: int, K: int, N: int,
                            kmajor: bool, nmajor: bool) -> None:
    """A reused QuantWeight must describe the same call (recipe, format,
    E, K, N, the requested layouts) with buffers of at least the sizes
    mxsg_quantize_weight_sizes gives."""
    if (q.recipe, q.fmt, q.E, q.K, q.N) != (recipe, f, E, K, N):
        raise ValueError(f"out was made for recipe={q.recipe} fmt={q.fmt} E={q.E} K={q.K} N={q.N}, "
                         f"the call has recipe={recipe} fmt={f} E={E} K={K} N={N}")
    nb = quantize_weight_sizes(E, K, N, recipe, f)
    sdt = _scale_dtype(recipe)
    for want, codes, scales, i, name in ((kmajor, q.kmajor_codes, q.kmajor_scales, 0, "kmajor"),
                                         (nmajor, q.nmajor_codes, q.nmajor_scales, 2, "nmajor")):
        if want:
            _need(codes, nb[i], f"out.{name}_codes", torch.uint8)
            _need(scales, nb[i + 1], f"out.{name}_scales", sdt)
        elif codes is not None:
            raise ValueError(f"out holds {name} codes but the call asks for none")
    if recipe in ("tw", "nvfp4"):
        _need(q.amax, 4 * E, "out.amax", torch.float32)


@dataclasses.dataclass
class QuantWeight:
    recipe: str
    fmt: int
    E: int
    K: int
    N: int
    kmajor_codes: Optional[torch.Tensor] = None   # uint8 [E, N, K] (K/2 for e2m1; forward operand, pair-interleaved)
    kmajor_scales: Optional[torch.Tensor] = None
    nmajor_codes: Optional[torch.Tensor] = None   # uint8 [E, K, N] (N/2 for e2m1; dgrad operand, pair-interleaved)
    nmajor_scales: Optional[torch.Tensor] = None
    amax: Optional[torch.Tensor] = None


def quantize_weight(w: torch.Tensor, recipe: str, fmt, kmajor: bool = True, nmajor: bool = True,
                    state: Optional[DelayedState] = None, unit: int = 0,
                    out: Optional[QuantWeight] = None,
                    status: Optional[torch.Tensor] = None) -> QuantWeight:
    """Quantize expert weights [E, K, N] (mxsg_quantize_weight); ``status``
    (int32 [1], device) receives MXSG_STATUS_NONFINITE for NaN / Inf weights."""
    w = _bits16(w)
    _check_dev(w, status)
    E, K, N = w.shape
    f = FMT[fmt]
    dev = w.device
    q = out
    if q is not None:
        _check_quant_weight_out(q, recipe, f, E, K, N, kmajor, nmajor)
    else:
        q = QuantWeight(recipe, f, E, K, N)
        nb = quantize_weight_sizes(E, K, N, recipe, f)
        epb = elems_per_byte(f)
        if recipe in ("tw", "dl"):
            ks = ns = _buffer(nb[1], torch.float32, 0, dev)
        elif recipe == "block":
            ks = ns = _buffer(nb[1], torch.float32, N // 128, dev).view(E, K // 128, N // 128)
        elif recipe == "nvfp4":  # block codes [E, K/128, N, 8] / [E, N/128, K, 8], then fp32 [E]
            ks = _buffer(nb[1], torch.uint8, 0, dev)
            ns = _buffer(nb[3], torch.uint8, 0, dev)
        else:  # word-major per expert: [E, K/128, N, 4] and [E, N/128, K, 4]
            ks = _buffer(nb[1], torch.uint8, 0, dev).view(E, K // 128, N, 4)
            ns = _buffer(nb[3], torch.uint8, 0, dev).view(E, N // 128, K, 4)
        if kmajor:
            q.kmajor_codes = _buffer(nb[0], torch.uint8, K // epb, dev).view(E, N, K // epb)
            q.kmajor_scales = ks
        if nmajor:
            q.nmajor_codes = _buffer(nb[2], torch.uint8, N // epb, dev).view(E, K, N // epb)
            q.nmajor_scales = ns
        if recipe in ("tw", "nvfp4"):
            q.amax = torch.empty(E, dtype=torch.float32, device=dev)
    amax = q.amax
    dls = dli = None
    if recipe == "dl":
        if state is None:
            raise ValueError("recipe 'dl' needs a DelayedState")
        if not (0 <= unit and unit + E <= state.units):
            raise ValueError(f"units {unit}..{unit + E - 1} outside the state's {state.units} units")
        amax = state.amax[unit:unit + E]
        dls = state.scale[unit:unit + E]
        dli = state.inv[unit:unit + E]
    _lib.call("mxsg_quantize_weight", _ptr(w), E, K, N, RECIPES[recipe], f,
              _ptr(q.kmajor_codes), _ptr(q.kmajor_scales), _ptr(q.nmajor_codes),
              _ptr(q.nmajor_scales), _ptr(amax), _ptr(dls), _ptr(dli), _ptr(_status_word(status)),
              _stream())
    return q


def _check_gemm_buffers(mode, recipe, fa, E, M, K, N, group_ends, a, a_scales, lda, b, b_scales, ldb,
                        padded_starts, out) -> None:
    """Sizes and dtypes of every buffer of a grouped_mm call (the layouts of
    mxsg.h): codes, scales, group ends, padded starts and the output."""
    epb = 2 if fa == E2M1 else 1
    _need(group_ends, 4 * E, "group_ends", torch.int32)
    if mode == MODE_WGRAD:
        a_rows, b_rows = K, N                         # column-wise codes [K, lda], [N, ldb]
        a_units, b_units = (K, lda * epb), (N, ldb * epb)
        _need(padded_starts, 4 * (E + 1), "padded_starts", torch.int32)
        out_bytes, out_dt = 4 * E * K * N, torch.float32
    else:
        L = K if mode == MODE_FWD else N             # contraction elements
        J = N if mode == MODE_FWD else K
        a_rows, b_rows = M + (M & 1), E * J
        a_units, b_units = (M, L), (E * J, L)
        out_bytes, out_dt = 2 * M * J, torch.bfloat16
    _need(a, a_rows * lda, "A codes", torch.uint8)
    _need(b, b_rows * ldb, "B codes", torch.uint8)
    if recipe in ("tw", "dl"):
        _need(a_scales, 4, "A scales", torch.float32)
        _need(b_scales, 4 * (1 if mode == MODE_WGRAD else E), "B scales", torch.float32)
    elif recipe == "nvfp4":      # e4m3 block codes per 16 elements, then the fp32 tensor scale(s)
        _need(a_scales, a_units[0] * (a_units[1] // 16) + 4, "A scales", torch.uint8)
        _need(b_scales, b_units[0] * (b_units[1] // 16) + 4 * (1 if mode == MODE_WGRAD else E), "B scales",
              torch.uint8)
    else:
        blk, per = (128, 4) if recipe == "block" else (32, 1)
        sdt = torch.float32 if recipe == "block" else torch.uint8
        _need(a_scales, a_units[0] * (a_units[1] // blk) * per, "A scales", sdt)
        if recipe == "block" and mode != MODE_WGRAD:   # 128x128 weight tiles
            _need(b_scales, 4 * E * (K // 128) * (N // 128), "B scales", sdt)
        else:
            _need(b_scales, b_units[0] * (b_units[1] // blk) * per, "B scales", sdt)
    if out is not None:
        _need(out, out_bytes, "out", out_dt)


def grouped_mm(mode: int, recipe: str, fmt_a, fmt_b, E: int, M: int, K: int, N: int,
               group_ends: torch.Tensor, a: torch.Tensor, a_scales: torch.Tensor, lda: int,
               b: torch.Tensor, b_scales: torch.Tensor, ldb: int,
               padded_starts: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
               accumulate: bool = False, status: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Raw grouped GEMM call (mxsg_grouped_mm); see the helpers below.
    ``status`` (int32 [1], device) receives the MXSG_STATUS_ENDS_* bits."""
    _check_dev(group_ends, a, a_scales, b, b_scales, padded_starts, out, status)
    _check_gemm_buffers(mode, recipe, FMT[fmt_a], E, M, K, N, group_ends, a, a_scales, lda, b,
                        b_scales, ldb, padded_starts, out)
    dev = a.device
    if out is None:
        if mode == MODE_FWD:
            out = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        elif mode == MODE_DGRAD:
            out = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
        else:
            out = torch.empty(E, K, N, dtype=torch.float32, device=dev)
    _lib.call("mxsg_grouped_mm", mode, RECIPES[recipe], FMT[fmt_a], FMT[fmt_b], E, M, K, N,
              _ptr(group_ends), _ptr(padded_starts), _ptr(a), _ptr(a_scales), lda, _ptr(b),
              _ptr(b_scales), ldb, _ptr(out), int(bool(accumulate)), _ptr(_status_word(status)),
              _stream())
    return out


def batch_group_ends(E: int, m: int, device) -> torch.Tensor:
    """Group ends of a 3-D (batched) token operand [E, m, C], e.g. the
    shared-expert case: its [E*m, C] view is E equal groups with ends m, 2m,
    ..., E*m, so quantize_act and grouped_mm take it unchanged (int32 [E])."""
    return torch.arange(1, E + 1, dtype=torch.int32, device=device) * int(m)


def grouped_mm_fwd(qa: QuantAct, qw: QuantWeight, group_ends: torch.Tensor,
                   out: Optional[torch.Tensor] = None, status: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y [M, N] (bf16) = A_g @ W_g per group, from row-wise A and k-major W."""
    epb = elems_per_byte(qa.fmt)
    return grouped_mm(MODE_FWD, qa.recipe, qa.fmt, qw.fmt, qw.E, qa.M, qw.K, qw.N, group_ends,
                      qa.row_codes, qa.row_scales, qa.C // epb, qw.kmajor_codes, qw.kmajor_scales,
                      qw.K // epb, out=out, status=status)


def grouped_mm_dgrad(qdy: QuantAct, qw: QuantWeight, group_ends: torch.Tensor,
                     out: Optional[torch.Tensor] = None, status: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dA [M, K] (bf16) = dY_g @ W_g^T per group, from row-wise dY and n-major W."""
    epb = elems_per_byte(qdy.fmt)
    return grouped_mm(MODE_DGRAD, qdy.recipe, qdy.fmt, qw.fmt, qw.E, qdy.M, qw.K, qw.N, group_ends,
                      qdy.row_codes, qdy.row_scales, qdy.C // epb, qw.nmajor_codes, qw.nmajor_scales,
                      qw.N // epb, out=out, status=status)


def grouped_mm_wgrad(qa: QuantAct, qdy: QuantAct, group_ends: torch.Tensor,
                     out: Optional[torch.Tensor] = None, accumulate: bool = False,
                     status: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dW [E, K, N] (fp32) = A_g^T @ dY_g per group, from the column-wise operands."""
    E = int(group_ends.numel())
    epb = elems_per_byte(qa.fmt)
    return grouped_mm(MODE_WGRAD, qa.recipe, qa.fmt, qdy.fmt, E, qa.M, qa.C, qdy.C, group_ends,
                      qa.col_codes, qa.col_scales, qa.ld // epb, qdy.col_codes, qdy.col_scales,
                      qdy.ld // epb, padded_starts=qa.padded_starts, out=out, accumulate=accumulate,
                      status=status)


def cast_sweep(start_bits: int, n: int, fmt, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Codes of the fp32 bit patterns start_bits .. start_bits + n - 1 (mxsg_cast_sweep)."""
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device="cuda")
    _lib.call("mxsg_cast_sweep", start_bits & 0xFFFFFFFF, n, FMT[fmt], _ptr(out), _stream())
    return out


def swiglu(x: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The bf16 SwiGLU activation [M, C] of a gate/up output x [M, 2C]
    (mxsg_swiglu): the value nearest to silu(gate) * up, ties to even."""
    x = _bits16(x)
    _check_dev(x, out)
    M, C2 = x.shape
    if C2 % 16:
        raise ValueError("a gate/up output needs 2C columns with C a multiple of 8")
    C = C2 // 2
    if out is None:
        out = torch.empty(M, C, dtype=torch.bfloat16, device=x.device)
    _need(out, 2 * M * C, "out")
    if out.element_size() != 2:
        raise TypeError("out must be a 16-bit (bf16) tensor")
    _lib.call("mxsg_swiglu", _ptr(x), M, C, _ptr(out), _stream())
    return out


def sigmoid_sweep() -> torch.Tensor:
    """The device's fast-path fp32 sigmoid of every bf16 bit pattern
    (mxsg_sigmoid_sweep): float32 [65536]."""
    out = torch.empty(65536, dtype=torch.float32, device="cuda")
    _lib.call("mxsg_sigmoid_sweep", _ptr(out), _stream())
    return out


def stream_copy(src: torch.Tensor, dst: torch.Tensor) -> None:
    """Device copy of src's bytes into dst (mxsg_stream_copy): the HBM
    reference rate for the quantization passes."""
    _check_dev(src, dst)
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n:
        raise ValueError("dst is smaller than src")
    _lib.call("mxsg_stream_copy", _ptr(src), _ptr(dst), n, _stream())


def clock_probe(iters: int = 200000, blocks: int = 0) -> dict:
    """The engine clock under matrix-core load (mxsg_clock_probe): `blocks`
    workgroups (default 4 per compute unit) of bf16 MFMAs for `iters`
    rounds; returns the median, min and max over workgroups of core cycles
    per second, in MHz. Synchronizes the device."""
    if blocks <= 0:
        blocks = 4 * torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    out = torch.zeros(4 * blocks, dtype=torch.int64, device="cuda")
    khz = ctypes.c_int32(0)
    _lib.call("mxsg_wall_clock_rate_khz", ctypes.addressof(khz))
    _lib.call("mxsg_clock_probe", blocks, iters, _ptr(out), _stream())
    t = out.view(blocks, 4).cpu()
    if int(t[:, 2].sum()) != 0:
        raise RuntimeError("clock_probe: non-finite accumulation")
    cyc, ticks = t[:, 0].double(), t[:, 1].double().clamp(min=1)
    mhz = (cyc / (ticks / (khz.value * 1e3))) / 1e6
    return {"mhz_median": float(mhz.median()), "mhz_min": float(mhz.min()), "mhz_max": float(mhz.max()),
            "wall_clock_khz": int(khz.value), "blocks": blocks, "iters": iters}
