"""Delayed scaling over the Mixtral delayed-hybrid schedule (history 1024,
"max" algorithm, activations drifting in scale by 1.01x per step over 50
steps; e4m3 activations and weights, e5m2 output gradients), at reduced
tensor sizes: the state logic does not depend on them.

* every step: codes, scales, recorded amaxes and the whole state (history,
  position, scale, inverse) bit-identical to the oracle's replay;
* forward, dgrad and wgrad GEMMs within 1e-3 of the oracle at steps 0, 1,
  25 and 49;
* checkpoint / resume: the state saved after step 25, loaded into freshly
  created state buffers, and run to step 49 gives the same state and the
  same codes, bit for bit, as the uninterrupted run."""
import numpy as np
import pytest

from tests.gpu_helpers import (torch, gpu_available, to_dev_u16, to_dev, host, codes_host,
                               bf16_host_f64, assert_bits_equal)
from oracle import quant as OQ
from oracle import formats as OF
from oracle import gemm as OG
from oracle.delayed import DelayedState as OracleDelayed
from mx_scaled_grouped_amd import workloads as W

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="no GPU")]

SIZES = [130, 0, 257, 64, 1, 300, 128, 95]   # 8 experts, ragged, one empty
K, N = 256, 384
STEPS = 50
GEMM_STEPS = (0, 1, 25, 49)
SEED = 140


def _api():
    from mx_scaled_grouped_amd import api
    return api


def _inputs(step):
    """Activations drift by 1.01x per step; weights fixed; dY fresh per step."""
    R = sum(SIZES)
    x = W.normal_bf16(SEED, 0, (R, K), std=1.01 ** step, step=step)
    w = W.normal_bf16(SEED, 1, (len(SIZES), K, N), std=0.02)
    dy = W.normal_bf16(SEED, 2, (R, N), std=2.0 ** -10, step=step)
    return x, w, dy


class Run:
    """Device side of the schedule: units 0 = x, 1..E = weights (e4m3 state);
    unit 0 = dY (e5m2 state)."""

    def __init__(self):
        api = _api()
        self.E = len(SIZES)
        self.st_f = api.DelayedState.create(1 + self.E, 0, 1024)
        self.st_g = api.DelayedState.create(1, 1, 1024)
        self.ge = to_dev(W.group_ends_from_sizes(SIZES))

    def step(self, t):
        api = _api()
        x, w, dy = _inputs(t)
        qx = api.quantize_act(to_dev_u16(x), "dl", 0, self.ge, rowwise=True, colwise=True,
                              state=self.st_f, unit=0)
        qw = api.quantize_weight(to_dev_u16(w), "dl", 0, state=self.st_f, unit=1)
        qd = api.quantize_act(to_dev_u16(dy), "dl", 1, self.ge, rowwise=True, colwise=True,
                              state=self.st_g, unit=0)
        out = {"qx": qx, "qw": qw, "qd": qd, "amax_f": host(self.st_f.amax).copy(),
               "amax_g": host(self.st_g.amax).copy()}
        if t in GEMM_STEPS:
            out["y"] = api.grouped_mm_fwd(qx, qw, self.ge)
            out["da"] = api.grouped_mm_dgrad(qd, qw, self.ge)
            out["dw"] = api.grouped_mm_wgrad(qx, qd, self.ge)
        self.st_f.update()
        self.st_g.update()
        return out


def _state(run):
    return {f"{n}.{k}": v.numpy() for n, st in (("f", run.st_f), ("g", run.st_g))
            for k, v in st.state_dict().items()}


def _check_step(t, got, ref_f, ref_g):
    ge = W.group_ends_from_sizes(SIZES)
    x, w, dy = _inputs(t)
    E = len(SIZES)
    rx = OQ.quantize_act(x, "dl", OF.E4M3, ge, rowwise=True, colwise=True, dl_scale=ref_f.scale(0))
    rw = OQ.quantize_weight(w, "dl", OF.E4M3, dl_scale=(ref_f.s[1:1 + E], ref_f.inv[1:1 + E]))
    rd = OQ.quantize_act(dy, "dl", OF.E5M2, ge, rowwise=True, colwise=True, dl_scale=ref_g.scale(0))
    R = x.shape[0]
    assert_bits_equal(codes_host(got["qx"].row_codes, R), rx["row_codes"], f"step {t} x codes")
    P = rx["padded_starts"]
    assert_bits_equal(codes_host(got["qx"].col_codes)[:, :P[-1]], rx["col_codes"], f"step {t} x col codes")
    assert_bits_equal(codes_host(got["qd"].row_codes, R), rd["row_codes"], f"step {t} dy codes")
    assert_bits_equal(codes_host(got["qd"].col_codes)[:, :P[-1]], rd["col_codes"], f"step {t} dy col codes")
    assert_bits_equal(codes_host(got["qw"].kmajor_codes), rw["kmajor_codes"], f"step {t} w k-major")
    assert_bits_equal(codes_host(got["qw"].nmajor_codes), rw["nmajor_codes"], f"step {t} w n-major")
    assert_bits_equal(host(got["qw"].kmajor_scales), rw["kmajor_scales"], f"step {t} w scales")
    assert_bits_equal(host(got["qx"].row_scales), rx["row_scales"], f"step {t} x scale")
    assert_bits_equal(got["amax_f"], np.concatenate([rx["amax"], rw["amax"]]), f"step {t} amax e4m3")
    assert_bits_equal(got["amax_g"], rd["amax"], f"step {t} amax e5m2")
    if "y" in got:
        A = OG.deq_act_rows(rx["row_codes"], rx["row_scales"], "dl", OF.E4M3)
        D = OG.deq_act_rows(rd["row_codes"], rd["row_scales"], "dl", OF.E5M2)
        y = OG.round_bf16(OG.grouped_fwd(A, OG.deq_weight(rw, "dl", OF.E4M3, "k"), ge))
        da = OG.round_bf16(OG.grouped_dgrad(D, OG.deq_weight(rw, "dl", OF.E4M3, "n"), ge))
        At = OG.unpad_cols(OG.deq_act_cols(rx["col_codes"], rx["col_scales"], "dl", OF.E4M3), P, ge)
        Dt = OG.unpad_cols(OG.deq_act_cols(rd["col_codes"], rd["col_scales"], "dl", OF.E5M2), P, ge)
        dw = OG.round_f32(OG.grouped_wgrad(At, Dt, ge, E))
        for what, g, r in (("fwd", bf16_host_f64(got["y"]), y), ("dgrad", bf16_host_f64(got["da"]), da),
                           ("wgrad", host(got["dw"]).astype(np.float64), dw)):
            e = OG.rel_fro(g, r)
            assert e <= 1e-3, f"step {t} {what}: rel err {e:.3e}"
    ref_f.update(np.concatenate([rx["amax"], rw["amax"]]))
    ref_g.update(rd["amax"])


def _defined_codes(got):
    """The written parts of a step's codes: R rows (the pad row of an odd
    row count is never written) and the columns below the last padded start."""
    R = sum(SIZES)
    rp = int(host(got["qx"].padded_starts)[-1])
    return [("x codes", codes_host(got["qx"].row_codes, R)),
            ("x column codes", codes_host(got["qx"].col_codes)[:, :rp]),
            ("w k-major codes", codes_host(got["qw"].kmajor_codes)),
            ("w n-major codes", codes_host(got["qw"].nmajor_codes)),
            ("dy codes", codes_host(got["qd"].row_codes, R)),
            ("dy column codes", codes_host(got["qd"].col_codes)[:, :rp])]


def test_fifty_steps_and_resume():
    E = len(SIZES)
    ref_f = OracleDelayed(1 + E, OF.E4M3, 1024)
    ref_g = OracleDelayed(1, OF.E5M2, 1024)
    run = Run()
    saved = None
    last = None
    for t in range(STEPS):
        print(f"delayed schedule step {t}", flush=True)
        got = run.step(t)
        _check_step(t, got, ref_f, ref_g)
        st = _state(run)
        assert_bits_equal(st["f.history"], ref_f.history, f"step {t} e4m3 history")
        assert_bits_equal(st["f.scale"], ref_f.s, f"step {t} e4m3 scale")
        assert_bits_equal(st["f.inv"], ref_f.inv, f"step {t} e4m3 inv")
        assert_bits_equal(st["g.history"], ref_g.history, f"step {t} e5m2 history")
        assert_bits_equal(st["g.scale"], ref_g.s, f"step {t} e5m2 scale")
        assert np.array_equal(st["f.pos"].astype(np.int64), ref_f.pos)
        assert np.array_equal(st["g.pos"].astype(np.int64), ref_g.pos)
        if t == 25:
            saved = {"f": run.st_f.state_dict(), "g": run.st_g.state_dict()}
        if t == STEPS - 1:
            last = (st, _defined_codes(got))
    # resume from the checkpoint in new state buffers
    run2 = Run()
    run2.st_f.load_state_dict(saved["f"])
    run2.st_g.load_state_dict(saved["g"])
    for t in range(26, STEPS):
        got2 = run2.step(t)
    st2 = _state(run2)
    for k in st2:
        assert_bits_equal(st2[k], last[0][k], f"resumed state {k}")
    for (what, g), (_, w) in zip(_defined_codes(got2), last[1]):
        assert_bits_equal(g, w, "resumed " + what)
