"""GPU parity of the fused SwiGLU-then-quantize pass (mxsg_quantize_act_swiglu)
against the oracle: the SwiGLU activation of oracle/swiglu.py (reproducible
fp32, rounded to bf16) quantized by the oracle's quantize_act. Codes, scales,
padded starts and the delayed amax must match bit for bit."""
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


def _f32_of_bits(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _bits_of_bf16_values(v):
    return (np.asarray(v, np.float64).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _case(seed, sizes, C, std):
    M = sum(sizes)
    h = W.normal_bf16(seed, 0, (M, 2 * C), std=std)
    h[0, 0] = 0xC2C8          # gate -100: silu -> -0
    h[0, 1] = 0x42C8          # gate +100: silu -> gate
    a = _bits_of_bf16_values(OS.swiglu_bf16(_f32_of_bits(h)))
    return h, a, W.group_ends_from_sizes(sizes)


@pytest.mark.parametrize("recipe,fmt", [("block", 0), ("block", 1), ("mx", 0), ("mx", 1), ("mx", 2)])
def test_swiglu_quant_matches_oracle(recipe, fmt):
    api = _api()
    sizes = [37, 0, 130, 1, 200]
    C = 384
    h, a, ge = _case(140 + fmt, sizes, C, 3.0)
    M = sum(sizes)
    print(f"quantize_act_swiglu {recipe} fmt={fmt} M={M} C={C}", flush=True)
    ref = OQ.quantize_act(a, recipe, FMT_OBJ[fmt], ge, rowwise=True, colwise=True)
    q = api.quantize_act(to_dev_u16(h), recipe, fmt, to_dev(ge), rowwise=True, colwise=True, swiglu=True)
    _compare_act(q, ref, recipe, M, C, True, True)


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
    a = _bits_of_bf16_values(OS.swiglu_bf16(_f32_of_bits(h)))
    print(f"quantize_act_swiglu mx row-only M={M} C={C}", flush=True)
    ref = OQ.quantize_act(a, "mx", FMT_OBJ[0], None, rowwise=True, colwise=False)
    q = api.quantize_act(to_dev_u16(h), "mx", 0, None, rowwise=True, colwise=False, swiglu=True)
    _compare_act(q, ref, "mx", M, C, True, False)


def test_swiglu_tensorwise_is_rejected():
    api = _api()
    h = W.normal_bf16(170, 0, (8, 256), std=1.0)
    with pytest.raises(Exception):
        api.quantize_act(to_dev_u16(h), "tw", 0, None, rowwise=True, swiglu=True)


@pytest.mark.parametrize("recipe,fmt", [("dl", 0), ("block", 0), ("mx", 0)])
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
