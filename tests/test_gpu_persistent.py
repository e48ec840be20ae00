"""Persistent quantized expert weights across gradient-accumulation
micro-batches (the single-grouped-weight PR's FP8 primary-weight and
gradient-accumulation-fusion rows): the weights change only at the
optimizer step, so both code layouts are quantized once per step and reused
by every micro-batch's forward and dgrad; wgrad accumulates each
micro-batch's dW into one fp32 main gradient; with delayed scaling the
weight units record their amax when quantized, the activation and gradient
units max-reduce theirs across the micro-batches, and the state is updated
once per optimizer step.

Checked against the oracle's replay over 2 optimizer steps x 3 micro-batches
(delayed hybrid and MX recipes): the reused weight codes are not modified
by any micro-batch, every code and scale is bit-exact, forward and dgrad of
every micro-batch and the accumulated wgrad of each step are within 1e-3,
and the delayed state after each step is bit-exact."""
import numpy as np
import pytest

from tests.gpu_helpers import (torch, gpu_available, to_dev_u16, to_dev, host, codes_host,
                               bf16_host_f64, assert_bits_equal, scales_host)
from oracle import quant as OQ
from oracle import formats as OF
from oracle import gemm as OG
from oracle.delayed import DelayedState as OracleDelayed
from mx_scaled_grouped_amd import workloads as W

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="no GPU")]

SIZES = [130, 0, 257, 64, 1]
K, N = 256, 384
MICRO = 3
STEPS = 2
SEED = 300


def _api():
    from mx_scaled_grouped_amd import api
    return api


def _inputs(step, mb):
    R = sum(SIZES)
    i = step * MICRO + mb
    x = W.normal_bf16(SEED, 0, (R, K), std=1.01 ** i, step=i)
    dy = W.normal_bf16(SEED, 2, (R, N), std=2.0 ** -10, step=i)
    return x, dy


def _weights(step):
    """The optimizer changes the weights between steps."""
    return W.normal_bf16(SEED, 1, (len(SIZES), K, N), std=0.02, step=step)


def _err(got, ref, what):
    e = OG.rel_fro(got, ref)
    assert e <= 1e-3, f"{what}: rel err {e:.3e}"


@pytest.mark.parametrize("recipe", ["dl", "mx"])
def test_persistent_weights_over_micro_batches(recipe):
    api = _api()
    E = len(SIZES)
    ge_h = W.group_ends_from_sizes(SIZES)
    ge = to_dev(ge_h)
    fa, fg = (0, 1) if recipe == "dl" else (0, 0)
    FA, FG = OF.E4M3, (OF.E5M2 if fg == 1 else OF.E4M3)
    if recipe == "dl":
        st_f = api.DelayedState.create(1 + E, fa, 1024)     # unit 0: x, 1..E: weights
        st_g = api.DelayedState.create(1, fg, 1024)         # unit 0: dY
        o_f, o_g = OracleDelayed(1 + E, FA, 1024), OracleDelayed(1, FG, 1024)
    dw = torch.empty(E, K, N, dtype=torch.float32, device="cuda")
    for step in range(STEPS):
        w = _weights(step)
        kw_w = dict(state=st_f, unit=1) if recipe == "dl" else {}
        qw = api.quantize_weight(to_dev_u16(w), recipe, fa, **kw_w)      # once per optimizer step
        snap = [t.clone() for t in (qw.kmajor_codes, qw.nmajor_codes, qw.kmajor_scales, qw.nmajor_scales)]
        # oracle weight codes with the scales the state holds at this step
        if recipe == "dl":
            ws, wi = o_f.s[1:].copy(), o_f.inv[1:].copy()
            rw = OQ.quantize_weight(w, "dl", FA, dl_scale=(ws, wi))
            xs, gs = o_f.scale(0), o_g.scale(0)
        else:
            rw = OQ.quantize_weight(w, "mx", FA)
        assert_bits_equal(codes_host(qw.kmajor_codes), rw["kmajor_codes"], "weight k-major codes")
        assert_bits_equal(codes_host(qw.nmajor_codes), rw["nmajor_codes"], "weight n-major codes")
        Wk = OG.deq_weight(rw, recipe, FA, "k")
        Wn = OG.deq_weight(rw, recipe, FA, "n")
        ref_dw = np.zeros((E, K, N))
        amax_x = amax_g = np.float32(0)
        for mb in range(MICRO):
            x, dy = _inputs(step, mb)
            print(f"persistent {recipe}: step {step} micro-batch {mb}", flush=True)
            kx = dict(state=st_f, unit=0) if recipe == "dl" else {}
            kg = dict(state=st_g, unit=0) if recipe == "dl" else {}
            qx = api.quantize_act(to_dev_u16(x), recipe, fa, ge, rowwise=True, colwise=True, **kx)
            qd = api.quantize_act(to_dev_u16(dy), recipe, fg, ge, rowwise=True, colwise=True, **kg)
            y = api.grouped_mm_fwd(qx, qw, ge)
            da = api.grouped_mm_dgrad(qd, qw, ge)
            api.grouped_mm_wgrad(qx, qd, ge, out=dw, accumulate=mb > 0)
            # oracle side of the micro-batch
            if recipe == "dl":
                rx = OQ.quantize_act(x, "dl", FA, ge_h, rowwise=True, colwise=True, dl_scale=xs)
                rd = OQ.quantize_act(dy, "dl", FG, ge_h, rowwise=True, colwise=True, dl_scale=gs)
                amax_x = max(amax_x, np.float32(np.asarray(rx["amax"]).reshape(-1)[0]))
                amax_g = max(amax_g, np.float32(np.asarray(rd["amax"]).reshape(-1)[0]))
            else:
                rx = OQ.quantize_act(x, "mx", FA, ge_h, rowwise=True, colwise=True)
                rd = OQ.quantize_act(dy, "mx", FG, ge_h, rowwise=True, colwise=True)
            R = x.shape[0]
            assert_bits_equal(codes_host(qx.row_codes, R), rx["row_codes"], "activation codes")
            assert_bits_equal(codes_host(qd.row_codes, R), rd["row_codes"], "gradient codes")
            assert_bits_equal(scales_host(qx.row_scales, recipe), rx["row_scales"], "activation scales")
            A = OG.deq_act_rows(rx["row_codes"], rx["row_scales"], recipe, FA)
            D = OG.deq_act_rows(rd["row_codes"], rd["row_scales"], recipe, FG)
            _err(bf16_host_f64(y), OG.round_bf16(OG.grouped_fwd(A, Wk, ge_h)), f"forward {step}.{mb}")
            _err(bf16_host_f64(da), OG.round_bf16(OG.grouped_dgrad(D, Wn, ge_h)), f"dgrad {step}.{mb}")
            P = rx["padded_starts"]
            At = OG.unpad_cols(OG.deq_act_cols(rx["col_codes"], rx["col_scales"], recipe, FA), P, ge_h)
            Dt = OG.unpad_cols(OG.deq_act_cols(rd["col_codes"], rd["col_scales"], recipe, FG), P, ge_h)
            ref_dw = OG.grouped_wgrad(At, Dt, ge_h, E, init=ref_dw)
            # the reused weight operand is read-only for the micro-batches
            for a, b in zip(snap, (qw.kmajor_codes, qw.nmajor_codes, qw.kmajor_scales, qw.nmajor_scales)):
                assert torch.equal(a, b), "a micro-batch modified the persistent weight codes"
        got_dw = host(dw).astype(np.float64)
        _err(got_dw, ref_dw, f"accumulated wgrad step {step}")
        assert not got_dw[1].any(), "empty expert"
        if recipe == "dl":
            # recorded amax: max over the micro-batches (activations, gradients), the weights once
            w_amax = [OQ.amax_of(OQ.bf16_to_f32(w[e])) for e in range(E)]
            assert_bits_equal(host(st_f.amax), np.array([amax_x] + w_amax, np.float32), "e4m3 amax")
            assert_bits_equal(host(st_g.amax), np.array([amax_g], np.float32), "e5m2 amax")
            st_f.update()
            st_g.update()
            o_f.update(np.array([amax_x] + w_amax, np.float32))
            o_g.update(np.array([amax_g], np.float32))
            for gpu, ora, tag in ((st_f, o_f, "e4m3"), (st_g, o_g, "e5m2")):
                assert_bits_equal(host(gpu.history), ora.history, tag + " history")
                assert_bits_equal(host(gpu.scale), ora.s, tag + " scale")
                assert_bits_equal(host(gpu.inv), ora.inv, tag + " inv")
                assert np.array_equal(host(gpu.pos).astype(np.int64), ora.pos), tag + " pos"
