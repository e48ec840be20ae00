"""GPU parity of the NVFP4 recipe (e2m1 elements, an e4m3 scale per 16
contraction elements, an fp32 scale per tensor unit) against the oracle:

* quantization: codes, e4m3 block codes, tensor scales, padded starts and
  amax bit for bit, for row-wise and per-group column-wise token tensors
  (edge group sizes, gathered rows, the fused SwiGLU input) and both weight
  layouts;
* grouped GEMM (f16 MFMAs on exactly dequantized operands): bit-exact on
  operands whose every partial sum is exact in fp32 (power-of-two block and
  tensor scales), within 1e-3 on random operands, for forward, dgrad and
  wgrad (also accumulating);
* the whole path on ragged groups: SQNR against the bf16 GEMM within 0.1 dB
  of the oracle's own."""
import numpy as np
import pytest

from tests.gpu_helpers import torch, gpu_available, to_dev_u16, to_dev, host, assert_bits_equal, EDGE_SIZES
from oracle import quant as OQ
from oracle import formats as OF
from oracle import gemm as OG
from oracle import routing as OR
from oracle import swiglu as OS
from mx_scaled_grouped_amd import workloads as W

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="no GPU")]
NV = 2   # the e2m1 format code


def _api():
    from mx_scaled_grouped_amd import api
    return api


def _codes(api, t, rows=None):
    return host(api.unpack_nvfp4_codes(t, rows))


def _scales(api, t, rows, L, units=1):
    b, ts = api.nvfp4_scales(t, rows, L, units)
    return host(b), host(ts)


def _compare_act(api, q, ref, M, C, rowwise, colwise):
    if rowwise:
        assert_bits_equal(_codes(api, q.row_codes, M), ref["row_codes"], "row codes")
        b, ts = _scales(api, q.row_scales, M, C)
        assert_bits_equal(b[0], ref["row_scales"], "row block codes")
        assert_bits_equal(ts, ref["tensor_scale"], "row tensor scale")
    if colwise:
        P = host(q.padded_starts).astype(np.int64)
        assert np.array_equal(P, ref["padded_starts"]), (P, ref["padded_starts"])
        Rp = int(P[-1])
        assert_bits_equal(_codes(api, q.col_codes)[:, :Rp], ref["col_codes"], "column codes")
        b, ts = _scales(api, q.col_scales, C, q.ld)
        assert_bits_equal(b[0][:, :Rp // 16], ref["col_scales"], "column block codes")
        assert_bits_equal(ts, ref["tensor_scale"], "column tensor scale")
    assert_bits_equal(host(q.amax), ref["amax"], "amax")


@pytest.mark.parametrize("layout", ["row", "col", "both"])
def test_act_edge_groups(layout):
    api = _api()
    x, _, _, ge = W.small_case(501, EDGE_SIZES, 256, 128, outlier=True)
    M, C = x.shape
    row, col = layout in ("row", "both"), layout in ("col", "both")
    print(f"nvfp4 quantize_act {layout} M={M} C={C}", flush=True)
    ref = OQ.quantize_act(x, "nvfp4", OF.E2M1, ge, rowwise=row, colwise=col)
    q = api.quantize_act(to_dev_u16(x), "nvfp4", NV, to_dev(ge), rowwise=row, colwise=col)
    _compare_act(api, q, ref, M, C, row, col)


def test_act_wide_range_and_zero_blocks():
    """Blocks far below the tensor amax (tiny or zero block scales) and
    values saturating the e2m1 range."""
    api = _api()
    x = W.normal_bf16(502, 0, (300, 384), std=1.0)
    xf = OQ.bf16_to_f32(x)
    xf[:, :16] *= np.float32(1e-6)          # a block scale that rounds to e4m3 subnormals or zero
    xf[5:9, 16:32] = 0                      # zero blocks
    xf[7, 100] = np.float32(3e4)            # a large tensor amax
    x = W.bf16_bits(xf)
    ge = W.group_ends_from_sizes([100, 0, 200])
    ref = OQ.quantize_act(x, "nvfp4", OF.E2M1, ge, rowwise=True, colwise=True)
    q = api.quantize_act(to_dev_u16(x), "nvfp4", NV, to_dev(ge), rowwise=True, colwise=True)
    _compare_act(api, q, ref, 300, 384, True, True)


def test_act_gather_and_swiglu():
    api = _api()
    topk = W.routing_for(1)
    r = OR.route(topk.expert_ids, topk.n_experts)
    x = W.token_activation(1)
    rt = api.route(to_dev(topk.expert_ids), topk.n_experts)
    q = api.quantize_act(to_dev_u16(x), "nvfp4", NV, rt.group_ends, rowwise=True, colwise=True,
                         row_index=rt.row_index)
    a = x[r["row_index"]]
    ref = OQ.quantize_act(a, "nvfp4", OF.E2M1, r["group_ends"].astype(np.int32), rowwise=True, colwise=True)
    _compare_act(api, q, ref, a.shape[0], a.shape[1], True, True)
    # SwiGLU input: gate/up [M, 2C] -> the oracle activation, quantized
    h = W.normal_bf16(503, 0, (257, 512), std=2.0)
    act = (OS.swiglu_bf16(OQ.bf16_to_f32(h).astype(np.float64)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    ge = W.group_ends_from_sizes([57, 200])
    q = api.quantize_act(to_dev_u16(h), "nvfp4", NV, to_dev(ge), rowwise=True, colwise=True, swiglu=True)
    ref = OQ.quantize_act(act, "nvfp4", OF.E2M1, ge, rowwise=True, colwise=True)
    _compare_act(api, q, ref, 257, 256, True, True)


def test_weights():
    api = _api()
    w = W.normal_bf16(504, 1, (3, 256, 384), std=0.02)
    w[2] = W.bf16_bits(OQ.bf16_to_f32(w[2]) * np.float32(1e3))
    E, K, N = w.shape
    ref = OQ.quantize_weight(w, "nvfp4", OF.E2M1)
    q = api.quantize_weight(to_dev_u16(w), "nvfp4", NV)
    assert_bits_equal(_codes(api, q.kmajor_codes), ref["kmajor_codes"], "k-major codes")
    assert_bits_equal(_codes(api, q.nmajor_codes), ref["nmajor_codes"], "n-major codes")
    kb, kts = _scales(api, q.kmajor_scales, N, K, E)
    nb, nts = _scales(api, q.nmajor_scales, K, N, E)
    assert_bits_equal(kb, ref["kmajor_scales"], "k-major block codes")
    assert_bits_equal(nb, ref["nmajor_scales"], "n-major block codes")
    assert_bits_equal(kts, ref["tensor_scale"], "tensor scales")
    assert_bits_equal(nts, ref["tensor_scale"], "tensor scales (n-major)")
    assert_bits_equal(host(q.amax), ref["amax"], "amax")


# ---- grouped GEMM ----------------------------------------------------------

def _pow2_block_codes(rng, shape, lo, hi):
    """e4m3 codes of 2^j, j in [lo, hi] (exponent field j + 7, mantissa 0)."""
    return ((rng.integers(lo, hi + 1, size=shape) + 7) << 3).astype(np.uint8)


def _operand(api, codes, blocks, ts):
    """Device code bytes and scale buffer of logical codes [units*rows..., L]
    and block codes [units, rows, L/16]."""
    c = api.pack_nvfp4_codes(torch.from_numpy(np.ascontiguousarray(codes)).cuda())
    s = api.pack_nvfp4_scales(torch.from_numpy(np.ascontiguousarray(blocks)).cuda(),
                              torch.from_numpy(np.asarray(ts, np.float32)).cuda())
    return c, s


def _run_case(mode, sizes, K, N, seed, exact, accumulate_init=None):
    api = _api()
    rng = np.random.default_rng(seed)
    E = len(sizes)
    ge = W.group_ends_from_sizes(sizes)
    M = int(ge[-1])

    def codes(shape):
        if exact:
            return rng.integers(0, 16, size=shape).astype(np.uint8)
        v = rng.standard_normal(shape) * 3
        return OF.encode_sat_rne(v.astype(np.float32), OF.E2M1)

    def blocks(shape):
        if exact:
            return _pow2_block_codes(rng, shape, 0, 1)
        return OF.encode_sat_rne(np.abs(rng.standard_normal(shape) * 50).astype(np.float32) + 1, OF.E4M3)

    ts_a = np.float32(2.0 ** rng.integers(-4, 4)) if exact else np.float32(rng.uniform(0.01, 1))
    if mode in (0, 1):
        L, J = (K, N) if mode == 0 else (N, K)
        a, sa = codes((M, L)), blocks((1, M, L // 16))
        b, sb = codes((E, J, L)), blocks((E, J, L // 16))
        ts_b = (2.0 ** rng.integers(-4, 4, size=E) if exact else rng.uniform(0.01, 1, size=E)).astype(np.float32)
        ac, asc = _operand(api, a, sa, [ts_a])
        # the weight scale buffer holds E experts' codes [E, L/128, J, 8] one after another
        bc, bsc = _operand(api, b.reshape(E * J, L), sb, ts_b)
        A = OF.decode(a, OF.E2M1) * np.repeat(OF.decode(sa[0], OF.E4M3), 16, axis=1) * float(ts_a)
        Bw = OF.decode(b, OF.E2M1) * np.repeat(OF.decode(sb, OF.E4M3), 16, axis=2) * ts_b[:, None, None]
        Wd = Bw.transpose(0, 2, 1)                                   # [E, L, J]
        ref = OG.round_bf16(OG.grouped_fwd(A, Wd, ge))
        out = api.grouped_mm(mode, "nvfp4", NV, NV, E, M, K, N, to_dev(ge), ac, asc, L // 2, bc, bsc, L // 2)
        got = OG.bf16_bits_to_f64(host(out.view(torch.int16)).view(np.uint16))
    else:
        P = OQ.padded_starts(ge)
        ld = int(_api().padded_capacity(M, E))
        Rp = int(P[-1])
        mask = np.zeros(ld, bool)
        for g in range(E):
            mask[P[g]:P[g] + sizes[g]] = True
        a = np.where(mask[None, :], codes((K, ld)), 0).astype(np.uint8)
        d = np.where(mask[None, :], codes((N, ld)), 0).astype(np.uint8)
        sa, sd = blocks((1, K, ld // 16)), blocks((1, N, ld // 16))
        ts_d = np.float32(2.0 ** rng.integers(-4, 4)) if exact else np.float32(rng.uniform(0.01, 1))
        ac, asc = _operand(api, a, sa, [ts_a])
        dc, dsc = _operand(api, d, sd, [ts_d])
        At = OF.decode(a, OF.E2M1) * np.repeat(OF.decode(sa[0], OF.E4M3), 16, axis=1) * float(ts_a)
        Dt = OF.decode(d, OF.E2M1) * np.repeat(OF.decode(sd[0], OF.E4M3), 16, axis=1) * float(ts_d)
        init = accumulate_init(E, K, N) if accumulate_init else None
        ref = OG.round_f32(OG.grouped_wgrad(OG.unpad_cols(At[:, :Rp], P, ge), OG.unpad_cols(Dt[:, :Rp], P, ge), ge,
                                            E, init=init))
        out = None
        if init is not None:
            out = torch.from_numpy(init.astype(np.float32)).cuda()
        out = api.grouped_mm(mode, "nvfp4", NV, NV, E, M, K, N, to_dev(ge), ac, asc, ld // 2, dc, dsc, ld // 2,
                             padded_starts=to_dev(P.astype(np.int32)), out=out, accumulate=init is not None)
        got = host(out).astype(np.float64)
    return got, ref, ge


@pytest.mark.parametrize("mode", [0, 1, 2], ids=["fwd", "dgrad", "wgrad"])
def test_gemm_exact_integer(mode):
    sizes = [0, 1, 127, 300, 64]
    got, ref, _ = _run_case(mode, sizes, 256, 384, 600 + mode, exact=True)
    print(f"nvfp4 exact mode {mode}: max |diff| {np.max(np.abs(got - ref))}", flush=True)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("mode", [0, 1, 2], ids=["fwd", "dgrad", "wgrad"])
def test_gemm_random(mode):
    sizes = EDGE_SIZES
    got, ref, ge = _run_case(mode, sizes, 512, 256, 610 + mode, exact=False)
    e = OG.rel_fro(got, ref)
    print(f"nvfp4 random mode {mode}: rel err {e:.2e}", flush=True)
    assert e <= 1e-3
    if mode in (0, 1):
        st = OQ.group_starts(ge)
        for g in range(len(sizes)):
            if ge[g] > st[g]:
                assert OG.rel_fro(got[st[g]:ge[g]], ref[st[g]:ge[g]]) <= 1e-3, g


def test_wgrad_accumulate_and_empty_groups():
    rng = np.random.default_rng(7)
    init = lambda E, K, N: rng.standard_normal((E, K, N)).astype(np.float32).astype(np.float64)
    got, ref, _ = _run_case(2, [0, 200, 0, 77], 256, 256, 620, exact=True, accumulate_init=init)
    assert np.array_equal(got, ref)


def test_path_sqnr():
    """Quantize activations, weights and gradients with the device, run all
    three GEMMs; SQNR against the float64 GEMM of the bf16 operands equals
    the oracle's within 0.1 dB."""
    api = _api()
    sizes = [190, 0, 257, 64, 513, 1]
    a, w, dy, ge = W.small_case(630, sizes, 512, 384, outlier=True)
    dy = W.normal_bf16(1630, 5, dy.shape, std=2.0 ** -10)
    E, K, N = w.shape
    ged = to_dev(ge)
    qa = api.quantize_act(to_dev_u16(a), "nvfp4", NV, ged, rowwise=True, colwise=True)
    qd = api.quantize_act(to_dev_u16(dy), "nvfp4", NV, ged, rowwise=True, colwise=True)
    qw = api.quantize_weight(to_dev_u16(w), "nvfp4", NV)
    y = api.grouped_mm_fwd(qa, qw, ged)
    da = api.grouped_mm_dgrad(qd, qw, ged)
    dw = api.grouped_mm_wgrad(qa, qd, ged)
    ra = OQ.quantize_act(a, "nvfp4", OF.E2M1, ge, rowwise=True, colwise=True)
    rd = OQ.quantize_act(dy, "nvfp4", OF.E2M1, ge, rowwise=True, colwise=True)
    rw = OQ.quantize_weight(w, "nvfp4", OF.E2M1)
    sc = lambda r, k: (r[k], r["tensor_scale"])
    A = OG.deq_act_rows(ra["row_codes"], sc(ra, "row_scales"), "nvfp4", OF.E2M1)
    D = OG.deq_act_rows(rd["row_codes"], sc(rd, "row_scales"), "nvfp4", OF.E2M1)
    P = ra["padded_starts"]
    At = OG.unpad_cols(OG.deq_act_cols(ra["col_codes"], sc(ra, "col_scales"), "nvfp4", OF.E2M1), P, ge)
    Dt = OG.unpad_cols(OG.deq_act_cols(rd["col_codes"], sc(rd, "col_scales"), "nvfp4", OF.E2M1), P, ge)
    af, df, wf = (OQ.bf16_to_f32(v).astype(np.float64) for v in (a, dy, w))
    cases = {
        "fwd": (OG.bf16_bits_to_f64(host(y.view(torch.int16)).view(np.uint16)),
                OG.round_bf16(OG.grouped_fwd(A, OG.deq_weight(rw, "nvfp4", OF.E2M1, "k"), ge)),
                OG.grouped_fwd(af, wf, ge)),
        "dgrad": (OG.bf16_bits_to_f64(host(da.view(torch.int16)).view(np.uint16)),
                  OG.round_bf16(OG.grouped_dgrad(D, OG.deq_weight(rw, "nvfp4", OF.E2M1, "n"), ge)),
                  OG.grouped_dgrad(df, wf, ge)),
        "wgrad": (host(dw).astype(np.float64), OG.round_f32(OG.grouped_wgrad(At, Dt, ge, E)),
                  OG.grouped_wgrad(af, df, ge, E)),
    }
    for k, (got, ref, hp) in cases.items():
        assert OG.rel_fro(got, ref) <= 1e-3, k
        s_gpu, s_ora = OG.sqnr_db(hp, got), OG.sqnr_db(hp, ref)
        print(f"nvfp4 {k}: SQNR device {s_gpu:.2f} dB, oracle {s_ora:.2f} dB", flush=True)
        assert abs(s_gpu - s_ora) <= 0.1, k
