"""GPU parity of the SwiGLU kernels against the oracle's plain definition
(oracle/swiglu.py: the bf16 value nearest to silu(g) * u, from float64 and,
near bf16 midpoints, exact decimal arithmetic).

* the device's fast fp32 sigmoid is within the 2^-21 relative error its
  fp64 fallback threshold assumes, on every bf16 gate with |g| <= 64;
* the plain activation (mxsg_swiglu) equals the oracle bit for bit on every
  bf16 gate pattern against several up values, on products that are exact
  bf16 midpoints, and on special values;
* the fused SwiGLU quantization (mxsg_quantize_act_swiglu) gives the codes,
  scales, padded starts and amax of the oracle's quantize_act applied to the
  oracle activation, for every recipe, bit for bit."""
import numpy as np
import pytest

from tests.gpu_helpers import torch, FMT_OBJ, gpu_available, to_dev_u16, to_dev, host, assert_bits_equal
from tests.test_gpu_quant import _compare_act
from oracle import quant as OQ
from oracle import swiglu as OS
from mx_scaled_grouped_amd import workloads as W

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="no GPU")]


def _api():
    from mx_scaled_grouped_amd import api
    return api


def _f64_of_bits(b):
    with np.errstate(invalid="ignore"):
        return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _bits_of_bf16_values(v):
    with np.errstate(invalid="ignore"):
        return (np.asarray(v, np.float64).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _act_bits(h_bits):
    """Oracle activation [M, F] as bf16 bits from gate/up bits [M, 2F]."""
    return _bits_of_bf16_values(OS.swiglu_bf16(_f64_of_bits(h_bits)))


def _device_swiglu(h_bits):
    api = _api()
    y = api.swiglu(to_dev_u16(h_bits))
    return host(y.view(torch.int16)).view(np.uint16)


def _compare_activation(got, want, what):
    """Bit-exact, except that any NaN matches any NaN."""
    gv, wv = _f64_of_bits(got), _f64_of_bits(want)
    nan = np.isnan(wv)
    assert np.array_equal(np.isnan(gv), nan), f"{what}: NaN positions differ"
    bad = np.flatnonzero((got != want) & ~nan)
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at flat index {bad[0]}: " \
                          f"got {got.reshape(-1)[bad[0]]:#06x} want {want.reshape(-1)[bad[0]]:#06x}"


def test_sigmoid_within_the_fallback_bound():
    api = _api()
    sig = host(api.sigmoid_sweep()).astype(np.float64)
    g = _f64_of_bits(np.arange(65536, dtype=np.uint32).astype(np.uint16))
    keep = np.isfinite(g) & (np.abs(g) <= 64)
    ref = OS.sigmoid_f64(g[keep])
    rel = np.abs(sig[keep] - ref) / ref
    worst = float(rel.max())
    print(f"fast sigmoid: max relative error {worst:.3e} = {worst / 2.0 ** -23:.2f} x 2^-23 "
          f"at g = {g[keep][rel.argmax()]!r}", flush=True)
    assert worst <= 2.0 ** -21


def test_activation_every_gate_pattern():
    """All 65536 gate bit patterns (NaN, Inf, zeros, subnormals, huge) against
    up values of many magnitudes; bit-exact with the oracle."""
    rng = np.random.default_rng(4)
    gates = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(256, 256)
    blocks = []
    for scale in (1.0, 3.0, 1e-3, 1e3, 1e-30, 1e30, 1e-38, 3e38):
        u = W.bf16_bits(rng.standard_normal((256, 256)).astype(np.float32) * np.float32(scale))
        blocks.append(np.concatenate([gates, u], axis=1))
    for ubits in (0x3F80, 0xBF80, 0x0000, 0x8000, 0x3F81, 0x7F80):   # 1, -1, +-0, 1 + 2^-7, +inf
        blocks.append(np.concatenate([gates, np.full_like(gates, ubits)], axis=1))
    h = np.concatenate(blocks, axis=0)
    print(f"swiglu exhaustive gates: {h.shape}", flush=True)
    _compare_activation(_device_swiglu(h), _act_bits(h), "activation")


def test_activation_exact_midpoint_products():
    """g * u an exact bf16 midpoint with large g: the true value lies just
    inside |g u| and rounds toward zero (a float64-only evaluation would see
    a tie); plus random data in the normal range."""
    pairs = []
    for g in _f64_of_bits(np.arange(0x4210, 0x4780, 3, dtype=np.uint32).astype(np.uint16)):   # 36 .. 2^16
        for u in _f64_of_bits(np.arange(0x3F80, 0x4000, dtype=np.uint32).astype(np.uint16)):
            p = g * u
            q = float(OS._bf16_quantum(np.float64(p)))
            if (p % q) == q / 2:
                pairs.append((g, u))
    pairs = np.array(pairs[:8192])
    pairs = np.concatenate([pairs, pairs * [1, -1], pairs * [-1, 1]])
    n = (len(pairs) // 8) * 8
    g = _bits_of_bf16_values(pairs[:n, 0]).reshape(-1, 8)
    u = _bits_of_bf16_values(pairs[:n, 1]).reshape(-1, 8)
    rng = np.random.default_rng(8)
    rnd = W.bf16_bits((rng.standard_normal((512, 16)) * 4).astype(np.float32))
    h = np.concatenate([np.concatenate([g, u], axis=1), rnd], axis=0)
    print(f"swiglu midpoint products: {n} pairs", flush=True)
    _compare_activation(_device_swiglu(h), _act_bits(h), "activation")


def _case(seed, sizes, C, std):
    M = sum(sizes)
    h = W.normal_bf16(seed, 0, (M, 2 * C), std=std)
    h[0, 0] = 0xC2C8          # gate -100: silu -> -0
    h[0, 1] = 0x42C8          # gate +100: silu -> gate
    h[1, 2] = 0x4340          # gate 192
    h[1, C + 2] = 0x3F81      # 192 * (1 + 2^-7) = 193.5, a midpoint: rounds to 193
    return h, _act_bits(h), W.group_ends_from_sizes(sizes)


@pytest.mark.parametrize("recipe,fmt", [("tw", 0), ("tw", 1), ("block", 0), ("block", 1), ("mx", 0),
                                        ("mx", 1), ("mx", 2)])
def test_swiglu_quant_matches_oracle(recipe, fmt):
    api = _api()
    sizes = [37, 0, 130, 1, 200]
    C = 384
    h, a, ge = _case(140 + fmt, sizes, C, 3.0)
    M = sum(sizes)
    print(f"quantize_act_swiglu {recipe} fmt={fmt} M={M} C={C}", flush=True)
    ref = OQ.quantize_act(a, recipe, FMT_OBJ[fmt], ge, rowwise=True, colwise=True)
    q = api.quantize_act(to_dev_u16(h), recipe, fmt, to_dev(ge), rowwise=True, colwise=True, swiglu=True)
    _compare_act(q, ref, recipe, M, C, True, True)          # tensorwise: the activation's amax too


@pytest.mark.parametrize("fmt", [0, 1], ids=["e4m3", "e5m2"])
def test_swiglu_quant_delayed(fmt):
    api = _api()
    sizes = [64, 0, 77, 50]
    C = 256
    h, a, ge = _case(150 + fmt, sizes, C, 2.0)
    M = sum(sizes)
    st = api.DelayedState.create(1, fmt, 16)
    st.scale.fill_(0.125)
    st.inv.fill_(8.0)
    q = api.quantize_act(to_dev_u16(h), "dl", fmt, to_dev(ge), rowwise=True, colwise=True,
                         state=st, unit=0, swiglu=True)
    ref = OQ.quantize_act(a, "dl", FMT_OBJ[fmt], ge, rowwise=True, colwise=True,
                          dl_scale=(np.float32(0.125), np.float32(8.0)))
    _compare_act(q, ref, "dl", M, C, True, True)
    assert_bits_equal(host(st.amax), ref["amax"], "delayed amax")


def test_swiglu_row_only_large_rows():
    """Row-wise only, more rows than one tile column of the grid holds, a
    ragged last tile, and the streaming-load path (input above 256 MiB)."""
    api = _api()
    M, C = 4100, 16384                                   # 4100 x 32768 bf16 = 269 MB
    h = W.normal_bf16(160, 0, (M, 2 * C), std=4.0)
    a = _act_bits(h)
    print(f"quantize_act_swiglu mx row-only M={M} C={C}", flush=True)
    ref = OQ.quantize_act(a, "mx", FMT_OBJ[0], None, rowwise=True, colwise=False)
    q = api.quantize_act(to_dev_u16(h), "mx", 0, None, rowwise=True, colwise=False, swiglu=True)
    _compare_act(q, ref, "mx", M, C, True, False)


@pytest.mark.parametrize("recipe,fmt", [("tw", 0), ("dl", 0), ("block", 0), ("mx", 0)])
def test_swiglu_status_word(recipe, fmt):
    """The non-finite bit reports a NaN or Inf activation: a NaN gate, an
    infinite gate times a zero up value (NaN), and nothing for finite inputs."""
    api = _api()
    sizes = [100, 28]
    C = 128
    ge = to_dev(W.group_ends_from_sizes(sizes))
    kw = {}
    if recipe == "dl":
        kw = dict(state=api.DelayedState.create(1, fmt, 4), unit=0)
    for poison, expect in ((None, 0), ((5, 3, 0x7FC0, None), api.STATUS_NONFINITE),
                           ((77, 100, 0x7F80, 0x0000), api.STATUS_NONFINITE)):
        h = W.normal_bf16(180, 0, (sum(sizes), 2 * C), std=1.0)
        if poison is not None:
            r, c, gbits, ubits = poison
            h[r, c] = gbits
            if ubits is not None:
                h[r, C + c] = ubits
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        api.quantize_act(to_dev_u16(h), recipe, fmt, ge, rowwise=True, colwise=True, swiglu=True,
                         status=status, **kw)
        got = int(host(status)[0])
        assert got == expect, (poison, got, expect)
