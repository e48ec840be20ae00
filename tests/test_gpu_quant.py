"""GPU parity of the quantization kernels against the CPU oracle: codes and
scales must match bit for bit (including the zero fill of the padded
column-wise layout), on ragged groups that include empty groups and
sizes around the block lengths."""
import numpy as np
import pytest

from tests.gpu_helpers import (torch, EDGE_SIZES, FMT_OBJ, gpu_available, to_dev_u16, to_dev, host, codes_host, scales_host,
                               codes_of, assert_bits_equal)
from oracle import quant as OQ
from oracle import formats as OF
from oracle.delayed import DelayedState as OracleDelayed
from mx_scaled_grouped_amd import workloads as W

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="no GPU")]


def _api():
    from mx_scaled_grouped_amd import api
    return api


# ---------------------------------------------------------------------------
# the device cast, exhaustively

def _segments_check(codes_dev, start: int, fmt, label: str):
    """codes_dev: device uint8 codes of the consecutive fp32 patterns start..;
    every run of equal codes must agree with the oracle at both of its ends
    (both encoders are monotone in the value, so that covers every input)."""
    n = codes_dev.numel()
    c = codes_dev
    change = torch.nonzero(c[1:] != c[:-1]).flatten()
    ends = torch.cat([change, torch.tensor([n - 1], device=c.device)])
    starts = torch.cat([torch.tensor([0], device=c.device), change + 1])
    idx = torch.cat([starts, ends]).cpu().numpy().astype(np.int64)
    got = c[torch.from_numpy(idx).cuda()].cpu().numpy()
    bits = (np.uint64(start) + idx.astype(np.uint64)).astype(np.uint32)
    vals = bits.view(np.float32)
    want = OF.encode_sat_rne(vals, fmt)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{label}: cast mismatch at bits {bits[bad[0]]:#010x}: got {got[bad[0]]:#x} want {want[bad[0]]:#x}"
    return int(change.numel())


@pytest.mark.parametrize("fmt", [0, 1, 2], ids=["e4m3", "e5m2", "e2m1"])
def test_cast_exhaustive(fmt):
    """Every non-NaN fp32 input, both signs: the saturating RNE cast used by
    all quantizers equals the oracle's table-search encoder."""
    api = _api()
    chunk = 1 << 27
    for sign in (0, 0x80000000):
        lo = sign
        hi = sign + 0x7F800001          # up to and including +-inf
        s = lo
        while s < hi:
            n = min(chunk, hi - s)
            print(f"cast sweep fmt={fmt} start={s:#010x} n={n}", flush=True)
            codes = api.cast_sweep(s, n, fmt)
            _segments_check(codes, s, FMT_OBJ[fmt], f"fmt={fmt}")
            s += n


def test_stream_copy():
    """The reference copy moves every byte, including a size that ends
    inside the last workgroup."""
    import torch
    api = _api()
    for n in (16, 4096 + 48, 3 * (1 << 20) + 16 * 7):
        src = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda")
        dst = torch.zeros(n + 64, dtype=torch.uint8, device="cuda")
        api.stream_copy(src, dst)
        torch.cuda.synchronize()
        assert torch.equal(dst[:n], src), n
        assert int(dst[n:].count_nonzero()) == 0, n


def test_clock_probe():
    """The engine clock under matrix-core load is a plausible engine clock
    (the chip's peak is 2.4 GHz) on every workgroup."""
    api = _api()
    c = api.clock_probe(iters=20000)
    print(f"clock probe: {c}", flush=True)
    assert c["wall_clock_khz"] > 0
    assert 300.0 <= c["mhz_min"] <= c["mhz_median"] <= c["mhz_max"] <= 2600.0, c


# ---------------------------------------------------------------------------
# token tensors

RECIPE_FMTS = [("tw", 0), ("tw", 1), ("block", 0), ("block", 1), ("mx", 0), ("mx", 1), ("mx", 2)]


def _compare_act(q, ref, recipe, M, C, rowwise, colwise):
    if rowwise:
        assert_bits_equal(codes_of(q.row_codes, q.fmt, M), ref["row_codes"], "row codes")
        assert_bits_equal(scales_host(q.row_scales, recipe), ref["row_scales"], "row scales")
    if colwise:
        P = host(q.padded_starts).astype(np.int64)
        assert np.array_equal(P, ref["padded_starts"]), (P, ref["padded_starts"])
        Rp = int(P[-1])
        assert_bits_equal(codes_of(q.col_codes, q.fmt)[:, :Rp], ref["col_codes"], "col codes")
        cs = scales_host(q.col_scales, recipe)
        if recipe in ("tw", "dl"):
            assert_bits_equal(cs, ref["col_scales"], "col scales")
        else:
            blk = 128 if recipe == "block" else 32
            assert_bits_equal(cs[:, :Rp // blk], ref["col_scales"], "col scales")
    if recipe == "tw":
        assert_bits_equal(host(q.amax), ref["amax"], "amax")


@pytest.mark.parametrize("recipe,fmt", RECIPE_FMTS)
@pytest.mark.parametrize("layout", ["row", "col", "both"])
def test_act_edge_groups(recipe, fmt, layout):
    api = _api()
    sizes = EDGE_SIZES
    x, _, _, ge = W.small_case(101, sizes, 256, 128, outlier=True)
    M, C = x.shape
    row = layout in ("row", "both")
    col = layout in ("col", "both")
    print(f"quantize_act {recipe} fmt={fmt} {layout} M={M} C={C}", flush=True)
    ref = OQ.quantize_act(x, recipe, FMT_OBJ[fmt], ge, rowwise=row, colwise=col)
    q = api.quantize_act(to_dev_u16(x), recipe, fmt, to_dev(ge), rowwise=row, colwise=col)
    _compare_act(q, ref, recipe, M, C, row, col)


@pytest.mark.parametrize("recipe,fmt", [("tw", 0), ("block", 0), ("mx", 1)])
def test_act_poisoned_outputs(recipe, fmt):
    """Outputs prefilled with 0xFF: every logical element and every padding
    code must be written."""
    api = _api()
    x, _, _, ge = W.small_case(102, [3, 0, 130, 0], 384, 128)
    M, C = x.shape
    ref = OQ.quantize_act(x, recipe, FMT_OBJ[fmt], ge, rowwise=True, colwise=True)
    q = api.quantize_act(to_dev_u16(x), recipe, fmt, to_dev(ge), rowwise=True, colwise=True)
    for t in (q.row_codes, q.col_codes, q.row_scales, q.col_scales, q.padded_starts):
        t.view(torch.uint8).fill_(0xFF)
    api.quantize_act(to_dev_u16(x), recipe, fmt, to_dev(ge), rowwise=True, colwise=True, out=q)
    _compare_act(q, ref, recipe, M, C, True, True)


def _routing_index(seed, T, M, drop):
    """A routed-row index: random tokens with repeats, out of order, never
    `drop`; the first entries hit both ends of x."""
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, T - 1, size=M)
    idx[idx >= drop] += 1
    idx[:2] = [T - 1, 0][:M]
    return idx.astype(np.int32)


@pytest.mark.parametrize("recipe,fmt", RECIPE_FMTS)
def test_act_gather(recipe, fmt):
    """Rows gathered inside the kernel (the dispatch permutation fused with
    quantization) are bit-exact against the oracle's gather-then-quantize,
    with a dropped token holding the largest value (tensorwise amax covers
    the routed rows only), on ragged groups including empty ones; and equal
    to the plain call on the explicitly gathered tensor."""
    api = _api()
    T, C = 300, 256
    x = W.normal_bf16(106, 0, (T, C))
    x[17, 3] = 0x4480                      # 1024.0 in a token nobody routes
    sizes = [0, 129, 1, 0, 260, 33]
    M = sum(sizes)
    idx = _routing_index(106, T, M, 17)
    ge = W.group_ends_from_sizes(sizes)
    print(f"quantize_act_gather {recipe} fmt={fmt} T={T} M={M}", flush=True)
    ref = OQ.quantize_act_gather(x, idx, recipe, FMT_OBJ[fmt], ge, rowwise=True, colwise=True)
    q = api.quantize_act(to_dev_u16(x), recipe, fmt, to_dev(ge), rowwise=True, colwise=True,
                         row_index=to_dev(idx))
    _compare_act(q, ref, recipe, M, C, True, True)
    p = api.quantize_act(to_dev_u16(x[idx.astype(np.int64)]), recipe, fmt, to_dev(ge), rowwise=True,
                         colwise=True)
    # defined parts only: the pad row of odd M and the columns past P_E are
    # not written
    Rp = int(ref["padded_starts"][-1])
    blk = {"block": 128, "mx": 32}.get(recipe)
    assert torch.equal(q.padded_starts, p.padded_starts)
    assert_bits_equal(codes_of(q.row_codes, fmt, M), codes_of(p.row_codes, fmt, M), "gathered row codes")
    assert torch.equal(q.row_scales, p.row_scales)
    assert_bits_equal(codes_of(q.col_codes, fmt)[:, :Rp], codes_of(p.col_codes, fmt)[:, :Rp],
                      "gathered column codes")
    if blk:
        assert_bits_equal(scales_host(q.col_scales, recipe)[:, :Rp // blk],
                          scales_host(p.col_scales, recipe)[:, :Rp // blk], "gathered column scales")
    else:
        assert torch.equal(q.col_scales, p.col_scales)


@pytest.mark.parametrize("fmt", [0, 1], ids=["e4m3", "e5m2"])
def test_act_gather_delayed(fmt):
    """Delayed scaling on gathered rows: codes from the state's scale, and the
    amax recorded in the state is that of the routed rows."""
    api = _api()
    T, C = 200, 384
    x = W.normal_bf16(107, 0, (T, C), std=3.0)
    x[5, 0] = 0x4600                       # 8192.0, dropped
    sizes = [64, 0, 77, 50]
    M = sum(sizes)
    idx = _routing_index(107, T, M, 5)
    ge = W.group_ends_from_sizes(sizes)
    st = api.DelayedState.create(1, fmt, 16)
    st.scale.fill_(0.125)
    st.inv.fill_(8.0)
    q = api.quantize_act(to_dev_u16(x), "dl", fmt, to_dev(ge), rowwise=True, colwise=True,
                         state=st, unit=0, row_index=to_dev(idx))
    ref = OQ.quantize_act_gather(x, idx, "dl", FMT_OBJ[fmt], ge, rowwise=True, colwise=True,
                                 dl_scale=(np.float32(0.125), np.float32(8.0)))
    _compare_act(q, ref, "dl", M, C, True, True)
    assert_bits_equal(host(st.amax), ref["amax"], "delayed amax")


def test_act_gather_empty_and_clamped():
    """M = 0 writes only the scales; indices outside [0, T) read a clamped
    row instead of faulting (the documented guard, not a supported use)."""
    api = _api()
    T, C = 40, 128
    x = W.normal_bf16(108, 0, (T, C))
    ge = W.group_ends_from_sizes([0, 0])
    q = api.quantize_act(to_dev_u16(x), "tw", 0, to_dev(ge), rowwise=True, colwise=True,
                         row_index=to_dev(np.zeros(0, np.int32)))
    assert host(q.padded_starts).tolist() == [0, 0, 0]
    assert host(q.amax).tolist() == [0.0] and host(q.row_scales).tolist() == [1.0]
    idx = np.array([-5, 3, T + 7, T - 1], np.int32)
    ge = W.group_ends_from_sizes([4])
    q = api.quantize_act(to_dev_u16(x), "mx", 0, to_dev(ge), rowwise=True, colwise=False,
                         row_index=to_dev(idx))
    ref = OQ.quantize_act_gather(x, np.clip(idx, 0, T - 1), "mx", OF.E4M3, ge)
    _compare_act(q, ref, "mx", 4, C, True, False)


def test_act_empty_and_single_row():
    api = _api()
    for sizes in ([0], [0, 0, 0], [1], [0, 1, 0]):
        x, _, _, ge = W.small_case(103, sizes, 128, 128)
        M = x.shape[0]
        for recipe in ("block", "mx", "tw"):
            print(f"edge M={M} sizes={sizes} {recipe}", flush=True)
            ref = OQ.quantize_act(x, recipe, OF.E4M3, ge, rowwise=True, colwise=True)
            q = api.quantize_act(to_dev_u16(x), recipe, 0, to_dev(ge), rowwise=True, colwise=True)
            _compare_act(q, ref, recipe, M, 128, True, True)


def test_act_wide_and_many_groups():
    """More than 64 groups (the group scan runs in passes of 64) and C > 128."""
    api = _api()
    rng = np.random.default_rng(5)
    sizes = list(rng.integers(0, 40, size=150))
    x, _, _, ge = W.small_case(104, sizes, 640, 128)
    for recipe in ("block", "mx", "tw"):
        print(f"many groups {recipe} M={x.shape[0]}", flush=True)
        ref = OQ.quantize_act(x, recipe, OF.E4M3, ge, rowwise=True, colwise=True)
        q = api.quantize_act(to_dev_u16(x), recipe, 0, to_dev(ge), rowwise=True, colwise=True)
        _compare_act(q, ref, recipe, x.shape[0], 640, True, True)


def test_act_special_values():
    """Zeros, signed zeros, bf16 subnormals and values that saturate."""
    api = _api()
    M, C = 96, 256
    x = W.normal_bf16(105, 0, (M, C))
    x[0, :] = 0
    x[1, :] = 0x8000                       # -0
    # bf16 subnormals next to normal values (a unit made only of values this
    # small has fmax/amax beyond float32, outside the contract)
    x[2, 0:256:2] = 0x0001                 # smallest bf16 subnormal
    x[3, 1:256:4] = 0x8005
    x[5, 5] = 0x7F7F                       # bf16 max
    x[4, 7] = 0x4780                       # 65536
    ge = W.group_ends_from_sizes([50, 46])
    for recipe in ("tw", "block", "mx"):
        for fmt in ((0, 1, 2) if recipe == "mx" else (0, 1)):
            print(f"special values {recipe} fmt={fmt}", flush=True)
            ref = OQ.quantize_act(x, recipe, FMT_OBJ[fmt], ge, rowwise=True, colwise=True)
            q = api.quantize_act(to_dev_u16(x), recipe, fmt, to_dev(ge), rowwise=True, colwise=True)
            _compare_act(q, ref, recipe, M, C, True, True)


# ---------------------------------------------------------------------------
# weights

@pytest.mark.parametrize("recipe,fmt", RECIPE_FMTS)
def test_weight_layouts(recipe, fmt):
    api = _api()
    w = W.normal_bf16(106, 0, (3, 256, 384), std=0.02)
    w[1, 7, 9] = W.bf16_bits(np.float32([3.0]))[0]           # one outlier in expert 1
    print(f"quantize_weight {recipe} fmt={fmt}", flush=True)
    ref = OQ.quantize_weight(w, recipe, FMT_OBJ[fmt])
    q = api.quantize_weight(to_dev_u16(w), recipe, fmt)
    assert_bits_equal(codes_of(q.kmajor_codes, fmt), ref["kmajor_codes"], "k-major codes")
    assert_bits_equal(codes_of(q.nmajor_codes, fmt), ref["nmajor_codes"], "n-major codes")
    assert_bits_equal(scales_host(q.kmajor_scales, recipe), ref["kmajor_scales"], "k-major scales")
    assert_bits_equal(scales_host(q.nmajor_scales, recipe), ref["nmajor_scales"], "n-major scales")
    if recipe == "tw":
        assert_bits_equal(host(q.amax), ref["amax"], "amax")


# Weight passes with k-major output launch their tiles in groups of row tiles
# (16, or 8 when the bf16 row stride is a multiple of 32 KiB). These shapes
# have several full groups and a partial last one, for both group sizes.
@pytest.mark.parametrize("shape,recipe,fmt", [
    ((2, 128 * 37, 256), "tw", 0), ((2, 128 * 37, 256), "block", 1), ((2, 128 * 37, 256), "mx", 0),
    ((2, 128 * 37, 256), "mx", 2), ((1, 128 * 19, 16384), "tw", 0), ((1, 128 * 11, 16384), "mx", 1)],
    ids=["g16-tw", "g16-block", "g16-mx", "g16-mxfp4", "g8-tw", "g8-mx"])
def test_weight_tile_groups(shape, recipe, fmt):
    api = _api()
    w = W.normal_bf16(108, 0, shape, std=0.02)
    w[-1, -1, -1] = W.bf16_bits(np.float32([-2.5]))[0]      # outlier in the last tile
    print(f"quantize_weight {shape} {recipe} fmt={fmt}", flush=True)
    ref = OQ.quantize_weight(w, recipe, FMT_OBJ[fmt])
    q = api.quantize_weight(to_dev_u16(w), recipe, fmt)
    assert_bits_equal(codes_of(q.kmajor_codes, fmt), ref["kmajor_codes"], "k-major codes")
    assert_bits_equal(codes_of(q.nmajor_codes, fmt), ref["nmajor_codes"], "n-major codes")
    assert_bits_equal(scales_host(q.kmajor_scales, recipe), ref["kmajor_scales"], "k-major scales")
    assert_bits_equal(scales_host(q.nmajor_scales, recipe), ref["nmajor_scales"], "n-major scales")
    # k-major only (the forward-only weight pass) uses the same tile order
    qk = api.quantize_weight(to_dev_u16(w), recipe, fmt, nmajor=False)
    assert_bits_equal(codes_of(qk.kmajor_codes, fmt), ref["kmajor_codes"], "k-major-only codes")


# ---------------------------------------------------------------------------
# delayed scaling

def test_delayed_steps_match_oracle():
    """Several steps of quantize (recording amax) + update, for an activation
    (with its column-wise copy) and a 3-expert weight, e4m3 and e5m2, with a
    short history so the window rolls over."""
    api = _api()
    L = 3
    st_dev = {0: api.DelayedState.create(4, 0, L), 1: api.DelayedState.create(1, 1, L)}
    st_ref = {0: OracleDelayed(4, OF.E4M3, L), 1: OracleDelayed(1, OF.E5M2, L)}
    sizes = [40, 0, 129]
    for step in range(6):
        grow = [1.0, 3.0, 0.5, 0.25, 2.0, 1.0][step]
        x = W.normal_bf16(107, 0, (sum(sizes), 256), std=grow, step=step)
        dy = W.normal_bf16(107, 1, (sum(sizes), 128), std=grow * 2 ** -10, step=step)
        w = W.normal_bf16(107, 2, (3, 256, 128), std=0.02 * grow, step=step)
        ge = W.group_ends_from_sizes(sizes)
        print(f"delayed step {step}", flush=True)
        # device
        qx = api.quantize_act(to_dev_u16(x), "dl", 0, to_dev(ge), rowwise=True, colwise=True,
                              state=st_dev[0], unit=0)
        qw = api.quantize_weight(to_dev_u16(w), "dl", 0, state=st_dev[0], unit=1)
        qd = api.quantize_act(to_dev_u16(dy), "dl", 1, to_dev(ge), rowwise=True, colwise=True,
                              state=st_dev[1], unit=0)
        # oracle
        rx = OQ.quantize_act(x, "dl", OF.E4M3, ge, rowwise=True, colwise=True, dl_scale=st_ref[0].scale(0))
        rw = OQ.quantize_weight(w, "dl", OF.E4M3, dl_scale=(st_ref[0].s[1:4], st_ref[0].inv[1:4]))
        rd = OQ.quantize_act(dy, "dl", OF.E5M2, ge, rowwise=True, colwise=True, dl_scale=st_ref[1].scale(0))
        _compare_act(qx, rx, "dl", x.shape[0], 256, True, True)
        _compare_act(qd, rd, "dl", dy.shape[0], 128, True, True)
        assert_bits_equal(codes_host(qw.kmajor_codes), rw["kmajor_codes"], "dl weight k-major")
        assert_bits_equal(codes_host(qw.nmajor_codes), rw["nmajor_codes"], "dl weight n-major")
        assert_bits_equal(host(qw.kmajor_scales), rw["kmajor_scales"], "dl weight scales")
        assert_bits_equal(host(st_dev[0].amax), np.concatenate([rx["amax"], rw["amax"]]), "recorded amax")
        assert_bits_equal(host(st_dev[1].amax), rd["amax"], "recorded amax dy")
        for f in (0, 1):
            st_dev[f].update()
        st_ref[0].update(np.concatenate([rx["amax"], rw["amax"]]))
        st_ref[1].update(rd["amax"])
        for f in (0, 1):
            assert_bits_equal(host(st_dev[f].scale), st_ref[f].s, "state scale")
            assert_bits_equal(host(st_dev[f].inv), st_ref[f].inv, "state inv")
            assert_bits_equal(host(st_dev[f].history), st_ref[f].history, "state history")
            assert np.array_equal(host(st_dev[f].pos), st_ref[f].pos)
            assert np.all(host(st_dev[f].amax) == 0)
