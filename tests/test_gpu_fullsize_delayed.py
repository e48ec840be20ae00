"""The Mixtral-shaped delayed-hybrid workload at full size over its whole
schedule (the Megatron-LM FP8-vs-BF16 MoE bug report reproduces with the
"max" amax algorithm and a history of 1024; here 50 steps, activations
scaled by 1.01^t at step t, fresh output gradients every step): the
benchmark's own Step and input generator, one full step per schedule step.

* every step: the delayed-scaling state after the step (history, position,
  scale, inverse) bit-exact against the oracle's replay, which takes every
  amax from the full tensors; codes and scales of sampled rows and of a
  128-wide column block of all four quantized token tensors bit-exact;
* steps 0, 1, 25 and 49: sampled forward, dgrad and wgrad outputs of both
  expert GEMMs within 1e-3 of the oracle and at the SQNR bar (the checks of
  the full-size sampled parity suite)."""
import numpy as np
import pytest

from tests.gpu_helpers import torch, gpu_available, assert_bits_equal
from tests import test_gpu_fullsize as FS
from oracle import quant as OQ
from oracle import formats as OF
from oracle import routing as OR
from oracle.delayed import DelayedState as ODelayed

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="no GPU")]

STEPS = 50
GEMM_STEPS = (0, 1, 25, 49)


def _codes_check(st, host_bits, kind, which, t):
    """Sampled row codes and one column block of a quantized token tensor."""
    step, ge = st["step"], st["ge"]
    gi = st["spec"].gemms.index(which)
    fmt = FS.FMT[step.fa if kind == "a" else step.fg]
    s, inv = st["scales"]["f" if kind == "a" else "g"]
    dls = (s[gi], inv[gi])
    x = host_bits[f"{kind}_{which}"]
    q = step.q[f"{kind}_{which}"]
    rows, _ = FS._row_sample(ge, 100 + t)
    r = OQ.quantize_act(x[rows], "dl", fmt, dl_scale=dls)
    assert_bits_equal(FS._codes(FS._take(FS._unpack(q.row_codes), (0, rows)), fmt), r["row_codes"],
                      f"step {t} {kind}_{which} row codes")
    assert_bits_equal(FS._np(q.row_scales)[:1], np.asarray(r["row_scales"], np.float32).reshape(-1)[:1],
                      f"step {t} {kind}_{which} scale")
    cols, _ = FS._block_sample(x.shape[1], 200 + t)
    cols = cols[:128]
    c = OQ.quantize_act(np.ascontiguousarray(x[:, cols]), "dl", fmt, ge, rowwise=False, colwise=True,
                        dl_scale=dls)
    P = c["padded_starts"]
    cc = FS._codes(FS._take(FS._unpack(q.col_codes), (0, cols)), fmt)
    assert_bits_equal(cc[:, :P[-1]], c["col_codes"], f"step {t} {kind}_{which} column codes")


@pytest.mark.timeout(1500)
def test_mixtral_delayed_full_schedule():
    import bench
    from mx_scaled_grouped_amd import api, workloads as W
    cid = 3
    spec, topk, ids, weights, _ = bench.make_inputs(cid, torch, W, api, sets=0)
    E, ng = spec.experts, len(spec.gemms)
    ro = OR.route(topk.expert_ids, E)
    step = bench.Step(torch, api, spec, ids, weights, spec.recipe)
    st = {"spec": spec, "step": step, "ge": ro["group_ends"], "row_index": ro["row_index"],
          "weights": weights, "recipe": "dl"}
    tokens = np.unique(ro["row_index"])
    sf = ODelayed(ng + ng * E, OF.E4M3, 1024)
    sg = ODelayed(ng, OF.E5M2, 1024)
    w_amax = []
    for which in spec.gemms:
        wb = FS._bits(weights[which])
        w_amax += [OQ.amax_of_bf16_bits(wb[e]) for e in range(E)]
        del wb
    g = torch.Generator(device="cuda")
    g.manual_seed(5000)
    for t in range(STEPS):
        data = bench.make_set(torch, g, cid, spec, topk.rows, t, step.rt.row_index)
        st["scales"] = {"f": (sf.s.copy(), sf.inv.copy()), "g": (sg.s.copy(), sg.inv.copy())}
        step.run(data)
        torch.cuda.synchronize()
        assert np.array_equal(FS._np(step.rt.row_index).astype(np.int64), ro["row_index"]), "routing"
        # the oracle's amaxes, from the full tensors (the gate/up input: the
        # token rows that are routed)
        xb = FS._bits(data["x_gu"])
        hb = {"a_gu": xb[ro["row_index"]], "a_dn": FS._bits(data["a_dn"]),
              "dy_gu": FS._bits(data["dy_gu"]), "dy_dn": FS._bits(data["dy_dn"])}
        a_amax = [OQ.amax_of_bf16_bits(xb[tokens]), OQ.amax_of_bf16_bits(hb["a_dn"])]
        g_amax = [OQ.amax_of_bf16_bits(hb["dy_gu"]), OQ.amax_of_bf16_bits(hb["dy_dn"])]
        sf.update(np.array(a_amax + w_amax, np.float32))
        sg.update(np.array(g_amax, np.float32))
        for gpu, ora, tag in ((step.st_f, sf, "e4m3 state"), (step.st_g, sg, "e5m2 state")):
            assert_bits_equal(FS._np(gpu.history), ora.history, f"step {t} {tag} history")
            assert_bits_equal(FS._np(gpu.scale), ora.s, f"step {t} {tag} scale")
            assert_bits_equal(FS._np(gpu.inv), ora.inv, f"step {t} {tag} inv")
            assert np.array_equal(FS._np(gpu.pos).astype(np.int64), ora.pos), f"step {t} {tag} pos"
        for kind in ("a", "dy"):
            for which in spec.gemms:
                _codes_check(st, hb, kind, which, t)
        print(f"[schedule] step {t}: state and codes bit-exact; e4m3 scale {sf.s[0]:.6g}, "
              f"e5m2 scale {sg.s[0]:.6g}", flush=True)
        if t in GEMM_STEPS:
            for which in spec.gemms:
                FS.forward_check(st, which, data, f"step {t}")
                FS.dgrad_check(st, which, data, f"step {t}")
                FS.wgrad_check(st, which, data, f"step {t}")
            print(f"[schedule] step {t}: GEMMs within 1e-3 and at the SQNR bar", flush=True)
        del data, hb, xb
