"""Host-side buffer checks of the torch binding (api.py): the C ABI takes
bare device pointers and cannot see buffer sizes, so the binding refuses a
reused output or an operand that is smaller than the call needs, or of the
wrong dtype, before anything reaches the library. These run on the CPU:
the checks look only at shapes and dtypes (the device check, which comes
first in the public calls, is bypassed by calling the checkers directly)."""
import os

import pytest

torch = pytest.importorskip("torch")

from mx_scaled_grouped_amd import _lib  # noqa: E402

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libmxsg.so not built")


def _api():
    from mx_scaled_grouped_amd import api
    return api


def _qa(api, recipe, fmt, M, C, E, rowwise=True, colwise=True):
    """A QuantAct with buffers of exactly the sizes the size query gives."""
    nb = api.quantize_act_sizes(M, C, recipe, fmt, E if colwise else 0)
    sdt = torch.uint8 if recipe == "mx" else torch.float32
    q = api.QuantAct(recipe, fmt, M, C)

    def buf(n, dt):
        return torch.empty(n // torch.empty(0, dtype=dt).element_size(), dtype=dt)
    if rowwise:
        q.row_codes, q.row_scales = buf(nb[0], torch.uint8), buf(nb[1], sdt)
    if colwise:
        q.ld = api.padded_capacity(M, E)
        q.col_codes, q.col_scales = buf(nb[2], torch.uint8), buf(nb[3], sdt)
        q.padded_starts = buf(nb[4], torch.int32)
    if recipe == "tw":
        q.amax = torch.empty(1)
    return q


@pytest.mark.parametrize("recipe", ["tw", "dl", "block", "mx"])
def test_reused_quant_act_is_checked(recipe):
    api = _api()
    M, C, E = 300, 256, 3
    q = _qa(api, recipe, 0, M, C, E)
    api._check_quant_act_out(q, recipe, 0, M, C, E, True, True)          # the matching call passes
    with pytest.raises(ValueError):
        api._check_quant_act_out(q, recipe, 0, M + 1, C, E, True, True)  # other M
    with pytest.raises(ValueError):
        api._check_quant_act_out(q, recipe, 1, M, C, E, True, True)      # other format
    with pytest.raises(ValueError):
        api._check_quant_act_out(q, recipe, 0, M, C, E + 5, True, True)  # other group count (ld)
    other = "mx" if recipe != "mx" else "block"
    with pytest.raises(ValueError):
        api._check_quant_act_out(q, other, 0, M, C, E, True, True)       # other recipe
    q.row_codes = q.row_codes[:-1]                                       # one byte short
    with pytest.raises(ValueError):
        api._check_quant_act_out(q, recipe, 0, M, C, E, True, True)
    q2 = _qa(api, recipe, 0, M, C, E, colwise=False)
    with pytest.raises(ValueError):
        api._check_quant_act_out(q2, recipe, 0, M, C, E, True, True)     # no column-wise buffers


@pytest.mark.parametrize("recipe", ["tw", "block", "mx"])
def test_reused_quant_weight_is_checked(recipe):
    api = _api()
    E, K, N = 2, 256, 384
    nb = api.quantize_weight_sizes(E, K, N, recipe, 0)
    sdt = torch.uint8 if recipe == "mx" else torch.float32
    isz = 1 if sdt == torch.uint8 else 4
    q = api.QuantWeight(recipe, 0, E, K, N, torch.empty(nb[0], dtype=torch.uint8),
                        torch.empty(nb[1] // isz, dtype=sdt), torch.empty(nb[2], dtype=torch.uint8),
                        torch.empty(nb[3] // isz, dtype=sdt),
                        torch.empty(E) if recipe == "tw" else None)
    api._check_quant_weight_out(q, recipe, 0, E, K, N, True, True)
    with pytest.raises(ValueError):
        api._check_quant_weight_out(q, recipe, 0, E, K, N + 128, True, True)
    with pytest.raises(ValueError):
        api._check_quant_weight_out(q, recipe, 0, E + 1, K, N, True, True)
    q.nmajor_scales = q.nmajor_scales[:-1]
    with pytest.raises(ValueError):
        api._check_quant_weight_out(q, recipe, 0, E, K, N, True, True)



def _gemm_args(api, mode, recipe, E=3, M=301, K=256, N=384):
    """Exactly sized operands of a grouped_mm call (host tensors)."""
    fa = 0
    ge = torch.zeros(E, dtype=torch.int32)
    if mode == api.MODE_WGRAD:
        qa = _qa(api, recipe, fa, M, K, E, rowwise=False)
        qd = _qa(api, recipe, fa, M, N, E, rowwise=False)
        a, sa, lda, b, sb, ldb = qa.col_codes, qa.col_scales, qa.ld, qd.col_codes, qd.col_scales, qd.ld
        ps = qa.padded_starts
        out = torch.empty(E, K, N)
    else:
        L = K if mode == api.MODE_FWD else N
        J = N if mode == api.MODE_FWD else K
        qa = _qa(api, recipe, fa, M, L, E, colwise=False)
        a, sa, lda = qa.row_codes, qa.row_scales, L
        nb = api.quantize_weight_sizes(E, K, N, recipe, fa)
        sdt = torch.uint8 if recipe == "mx" else torch.float32
        isz = 1 if sdt == torch.uint8 else 4
        b, sb, ldb = torch.empty(nb[0], dtype=torch.uint8), torch.empty(nb[1] // isz, dtype=sdt), L
        ps = None
        out = torch.empty(M, J, dtype=torch.bfloat16)
    return dict(mode=mode, recipe=recipe, fa=fa, E=E, M=M, K=K, N=N, group_ends=ge, a=a, a_scales=sa,
                lda=lda, b=b, b_scales=sb, ldb=ldb, padded_starts=ps, out=out)


@pytest.mark.parametrize("recipe", ["tw", "block", "mx"])
@pytest.mark.parametrize("mode", [0, 1, 2], ids=["fwd", "dgrad", "wgrad"])
def test_gemm_buffers_are_checked(mode, recipe):
    api = _api()
    kw = _gemm_args(api, mode, recipe)
    api._check_gemm_buffers(**kw)                                        # exact sizes pass
    for key in ("a", "b", "a_scales", "b_scales", "out", "group_ends"):
        bad = dict(kw)
        bad[key] = kw[key].reshape(-1)[:-1]                              # one element short
        with pytest.raises(ValueError):
            api._check_gemm_buffers(**bad)
    bad = dict(kw)
    bad["out"] = kw["out"].to(torch.float16 if mode != 2 else torch.bfloat16)
    with pytest.raises(TypeError):
        api._check_gemm_buffers(**bad)                                   # wrong output dtype
    if mode == 2:
        bad = dict(kw)
        bad["padded_starts"] = kw["padded_starts"][:-1]
        with pytest.raises(ValueError):
            api._check_gemm_buffers(**bad)
