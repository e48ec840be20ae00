"""The optional device status word: malformed group ends and non-finite
inputs set their MXSG_STATUS_* bits (mxsg.h), well-formed calls leave the
word at zero, and passing a status word does not change any output.

Malformed ends are clamped on the device (every access stays in bounds; the
numbers are then unspecified), so these calls only check the reported bits.
NaN / Inf inputs are outside the quantization contract: only the flag is
checked."""
import numpy as np
import pytest

from tests.gpu_helpers import torch, gpu_available, to_dev_u16, to_dev, host, assert_bits_equal
from mx_scaled_grouped_amd import workloads as W

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="no GPU")]

M, C = 300, 256


def _api():
    from mx_scaled_grouped_amd import api
    return api


def _status():
    return torch.zeros(1, dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("ends,bits", [
    ([100, 200, 300], 0),          # well formed
    ([100, 50, 300], 1),           # decreasing
    ([100, 400, 300], 1 | 2),      # past M, then decreasing
    ([-5, 100, 300], 1 | 2),       # negative (below the implicit 0 before the first group)
    ([100, 200, 250], 4),          # rows not covered exactly
    ([100, 200, 310], 2 | 4),      # last end past M
])
def test_group_ends_bits(ends, bits):
    api = _api()
    x = to_dev_u16(W.normal_bf16(120, 0, (M, C)))
    ge = to_dev(np.asarray(ends, np.int32))
    print(f"status ends={ends}", flush=True)
    st = _status()
    api.quantize_act(x, "block", 0, ge, rowwise=True, colwise=True, status=st)
    assert int(host(st)[0]) == bits
    # the grouped GEMM checks the same ends
    w = to_dev_u16(W.normal_bf16(120, 1, (3, C, 256), std=0.02))
    qa = api.quantize_act(x, "block", 0, to_dev(np.asarray([100, 200, 300], np.int32)), rowwise=True)
    qw = api.quantize_weight(w, "block", 0, nmajor=False)
    st2 = _status()
    api.grouped_mm_fwd(qa, qw, ge, status=st2)
    assert int(host(st2)[0]) == bits


def _with(bits, r, c, val):
    b = bits.copy()
    b[r, c] = val
    return b


@pytest.mark.parametrize("recipe", ["tw", "dl", "block", "mx"])
@pytest.mark.parametrize("bad", [0x7FC0, 0x7F80, 0xFF80], ids=["nan", "inf", "-inf"])
def test_nonfinite_input_bit(recipe, bad):
    api = _api()
    base = W.normal_bf16(121, 0, (M, C))
    ge = to_dev(np.asarray([100, 200, 300], np.int32))
    kw = {}
    if recipe == "dl":
        kw = dict(state=api.DelayedState.create(1, 0), unit=0)
    print(f"status nonfinite {recipe} {bad:#x}", flush=True)
    st = _status()
    api.quantize_act(to_dev_u16(base), recipe, 0, ge, rowwise=True, colwise=True, status=st, **kw)
    assert int(host(st)[0]) == 0, "finite input flagged"
    if recipe == "dl":
        kw = dict(state=api.DelayedState.create(1, 0), unit=0)
    st = _status()
    api.quantize_act(to_dev_u16(_with(base, 257, 131, bad)), recipe, 0, ge, rowwise=True, colwise=True,
                     status=st, **kw)
    assert int(host(st)[0]) == 8
    # weights
    w = W.normal_bf16(121, 1, (2, 256, 256), std=0.02)
    wkw = dict(state=api.DelayedState.create(2, 0), unit=0) if recipe == "dl" else {}
    st = _status()
    api.quantize_weight(to_dev_u16(w), recipe, 0, status=st, **wkw)
    assert int(host(st)[0]) == 0
    w[1, 200, 7] = bad
    wkw = dict(state=api.DelayedState.create(2, 0), unit=0) if recipe == "dl" else {}
    st = _status()
    api.quantize_weight(to_dev_u16(w), recipe, 0, status=st, **wkw)
    assert int(host(st)[0]) == 8


def test_status_word_changes_no_output():
    api = _api()
    x = to_dev_u16(W.normal_bf16(122, 0, (M, C)))
    ge = to_dev(np.asarray([100, 200, 300], np.int32))
    a = api.quantize_act(x, "mx", 0, ge, rowwise=True, colwise=True)
    b = api.quantize_act(x, "mx", 0, ge, rowwise=True, colwise=True, status=_status())
    for name in ("row_codes", "row_scales", "padded_starts"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    # column-wise: the defined columns (those past the last padded start are
    # not written)
    rp = int(host(a.padded_starts)[-1])
    assert torch.equal(api.unpack_codes(a.col_codes)[:, :rp], api.unpack_codes(b.col_codes)[:, :rp])
    assert torch.equal(api.unpack_mx_scales(a.col_scales)[:, :rp // 32],
                       api.unpack_mx_scales(b.col_scales)[:, :rp // 32])


def test_gathered_tensorwise_bit():
    """Tensorwise on routed rows: the amax pass over the gathered rows flags a
    NaN that a routed row carries, not one in a token nobody routes."""
    api = _api()
    T = 200
    xb = W.normal_bf16(123, 0, (T, C))
    idx = np.arange(M, dtype=np.int32) % 150          # tokens 150..199 are never routed
    ge = to_dev(np.asarray([100, 200, 300], np.int32))
    st = _status()
    api.quantize_act(to_dev_u16(_with(xb, 180, 3, 0x7FC0)), "tw", 0, ge, rowwise=True, status=st,
                     row_index=to_dev(idx))
    assert int(host(st)[0]) == 0
    st = _status()
    api.quantize_act(to_dev_u16(_with(xb, 42, 3, 0x7FC0)), "tw", 0, ge, rowwise=True, status=st,
                     row_index=to_dev(idx))
    assert int(host(st)[0]) == 8
