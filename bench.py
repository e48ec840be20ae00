#!/usr/bin/env python3
"""Benchmark of the quantized MoE expert grouped GEMM on one MI355X.

One step = the whole hot path over one batch of synthetic routed rows:
quantize activations (the gate/up input gathered from the token tensor
through the routing index inside the quantization kernel), expert weights
and output gradients, then the grouped GEMMs (forward, dgrad, wgrad for
both expert GEMMs) and, for delayed scaling, the amax-history update.

Default workload: Mixtral-8x7B-shaped experts (8 experts, hidden 4096,
ffn 14336, 8192 tokens top-2 = 16384 routed rows) with delayed scaling
(history 1024, max), e4m3 activations / weights and e5m2 gradients,
forward + dgrad + wgrad. ``--workload`` selects the other shapes.

Prints one JSON line (rank 0, N = 1). ``value`` is the GEMM FLOPs of a
step divided by the measured step time (quantization and the delayed
update included) in TFLOP/s.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

PEAK_FP8_TFLOPS = 5000.0       # MI355X dense FP8 MFMA
PEAK_FP4_TFLOPS = 10100.0      # MI355X dense FP4 / FP6 MFMA
PEAK_F16_TFLOPS = 2500.0       # MI355X dense FP16 / BF16 MFMA (the NVFP4 GEMM's arithmetic)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
GEMM_SOURCE = os.path.join(HERE, "mx_scaled_grouped_amd", "csrc", "gemm.hip")

WORKLOADS = {
    "mixtral-dl": 3,   # default: Mixtral shapes, delayed hybrid, fwd + dgrad + wgrad
    "mixtral-tw": 2,   # Mixtral shapes, tensorwise e4m3, forward only
    "deepseek-block": 4,
    "llama4-mx": 5,
    "llama4-mxfp4": 6,
    "llama4-nvfp4": 7,
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="mixtral-dl", choices=sorted(WORKLOADS))
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-swiglu", action="store_true",
                   help="skip the separate timing of the fused SwiGLU quantization")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device-to-device copy of MIB MiB (five times); "
                        "used to scale the HBM traffic counters")
    p.add_argument("--micro-batches", type=int, default=4, metavar="M",
                   help="also time optimizer steps of M micro-batches that quantize the weights once "
                        "and reuse them (0: skip)")
    p.add_argument("--cpu-sample-rows", type=int, default=1024)
    p.add_argument("--cpu-sample-cols", type=int, default=28672)
    return p.parse_args()


# ---------------------------------------------------------------------------
# synthetic inputs (generated on the GPU with torch's seeded generator; the
# distributions and routing follow mx_scaled_grouped_amd.workloads)

def _normal(torch, g, shape, std):
    """bf16 N(0, std^2) draws on the GPU from generator g."""
    t = torch.randn(shape, generator=g, device="cuda", dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(torch.bfloat16)


def _outliers(torch, g, cid, t):
    """Llama4-shaped workloads: 0.1% of the elements, drawn without
    replacement, multiplied by 50."""
    if cid not in (5, 6, 7):
        return t
    flat = t.view(-1)
    n = flat.numel()
    idx = torch.randperm(n, generator=g, device="cuda")[:max(1, n // 1000)]
    flat[idx] = (flat[idx].float() * 50.0).to(torch.bfloat16)
    return t


def make_inputs(cid, torch, W, api, sets=2):
    """Seeded inputs on the GPU: the top-k expert choices (device int32
    [T, k]), the weights and `sets` sets of activations and gradients. The
    routed rows of the gate/up input are gathered from the token rows by the
    step itself (routing kernel, then the gathering quantizer); `a_gu`, an
    explicit gathered copy made here with the device routing, is for callers
    that want the gathered tensor."""
    spec = W.SPECS[cid]
    topk = W.routing_for(cid)
    g = torch.Generator(device="cuda")
    g.manual_seed(1000 + cid)
    ids = torch.from_numpy(topk.expert_ids).to("cuda")
    row_token = api.route(ids, spec.experts).row_index
    gu_k, gu_n = spec.gemm_shape("gu")
    dn_k, dn_n = spec.gemm_shape("dn")
    weights = {"gu": _normal(torch, g, (spec.experts, gu_k, gu_n), 0.02)}
    if "dn" in spec.gemms:
        weights["dn"] = _normal(torch, g, (spec.experts, dn_k, dn_n), 0.02)
    sets_out = [make_set(torch, g, cid, spec, topk.rows, s, row_token) for s in range(sets)]
    return spec, topk, ids, weights, sets_out


def make_set(torch, g, cid, spec, R, s, row_token):
    """Input set s (activations scaled by 1.01^s for the delayed-scaling
    workload, whose activations drift from step to step)."""
    gu_k, gu_n = spec.gemm_shape("gu")
    dn_k, dn_n = spec.gemm_shape("dn")
    drift = 1.01 ** s if cid == 3 else 1.0
    x = _outliers(torch, g, cid, _normal(torch, g, (spec.tokens, gu_k), drift))
    # x_gu: the token tensor the step quantizes through the routing index
    # (gather fused into the quantization); a_gu: the same routed rows as
    # an explicit copy
    d = {"x_gu": x, "a_gu": x.index_select(0, row_token).contiguous()}
    if "dn" in spec.gemms:
        d["a_dn"] = _outliers(torch, g, cid, _normal(torch, g, (R, dn_k), drift))
    if "dgrad" in spec.modes:
        d["dy_gu"] = _normal(torch, g, (R, gu_n), 2.0 ** -10)
        if "dn" in spec.gemms:
            d["dy_dn"] = _normal(torch, g, (R, dn_n), 2.0 ** -10)
    return d


# ---------------------------------------------------------------------------

class Step:
    """One pass of the hot path; every call's duration is recorded with HIP
    events on the stream the kernels run on (torch's current stream)."""

    def __init__(self, torch, api, spec, ids, weights, recipe, gather=True):
        self.torch, self.api, self.spec, self.weights = torch, api, spec, weights
        self.ids = ids               # top-k expert choices, int32 [T, k] on the device
        # the routing buffers (group ends, routed row -> token), refilled by
        # the routing kernel at the start of every step
        self.rt = api.route(ids, spec.experts)
        self.ge = self.rt.group_ends
        self.gather = gather         # False: quantize the explicit gathered copy a_gu
        # "mxfp4" is the MX recipe with e2m1 elements for every operand;
        # NVFP4 has e2m1 elements only
        self.recipe = "mx" if recipe == "mxfp4" else recipe
        if recipe in ("mxfp4", "nvfp4"):
            self.fa = self.fw = self.fg = 2
        else:
            self.fa, self.fw = 0, 0
            self.fg = 1 if recipe == "dl" else 0     # hybrid: e5m2 gradients
        self.fp4 = recipe in ("mxfp4", "nvfp4")
        self.E = spec.experts
        self.bwd = "dgrad" in spec.modes
        self.q = {}        # reused quantized outputs
        self.out = {}      # reused GEMM outputs
        self.timing = None
        if recipe == "dl":
            # e4m3 units: a_gu, a_dn, then E per weight; e5m2 units: dy_gu, dy_dn
            ng = len(spec.gemms)
            self.st_f = api.DelayedState.create(ng + ng * self.E, 0, 1024)
            self.st_g = api.DelayedState.create(ng, 1, 1024)
        self.flops = {}
        self.bytes = {}

    def _t(self, name, fn):
        if self.timing is None:
            return fn()
        e0 = self.torch.cuda.Event(enable_timing=True)
        e1 = self.torch.cuda.Event(enable_timing=True)
        e0.record()
        r = fn()
        e1.record()
        self.timing.append((name, e0, e1))
        return r

    def run(self, data, timing=None):
        """One step: one batch through the whole path (weights quantized)."""
        self.optimizer_step([data], timing)

    def optimizer_step(self, datas, timing=None):
        """One optimizer step over len(datas) micro-batches: the expert
        weights change only at the optimizer step, so they are quantized
        (both layouts) once, before the first micro-batch, and every
        micro-batch reuses them; wgrad accumulates into the fp32 main
        gradient after the first micro-batch; the delayed-scaling state is
        updated once, after the last (its activation / gradient amaxes are
        then the maxima over the micro-batches)."""
        self.timing = timing
        for b, data in enumerate(datas):
            self._micro_batch(data, first=b == 0)
        if self.recipe == "dl":
            self._t("delayed_update", lambda: (self.st_f.update(), self.st_g.update()))
        self.timing = None

    def _micro_batch(self, data, first):
        api, spec, r = self.api, self.spec, self.recipe
        bwd = self.bwd
        self._t("route", lambda: api.route(self.ids, spec.experts, out=self.rt))
        for gi, which in enumerate(spec.gemms):
            K, N = spec.gemm_shape(which)
            a, w = data["a_" + which], self.weights[which]
            kw = {}
            if r == "dl":
                kw = dict(state=self.st_f, unit=gi)
            if which == "gu" and self.gather:
                # the routed rows are gathered from the tokens inside the kernel
                a = data["x_gu"]
                kw["row_index"] = self.rt.row_index
            qa = self._t(f"quant_a_{which}", lambda: api.quantize_act(
                a, r, self.fa, self.ge, rowwise=True, colwise=bwd, out=self.q.get("a_" + which), **kw))
            self.q["a_" + which] = qa
            kw = {}
            if r == "dl":
                kw = dict(state=self.st_f, unit=len(spec.gemms) + gi * self.E)
            if first:
                qw = self._t(f"quant_w_{which}", lambda: api.quantize_weight(
                    w, r, self.fw, kmajor=True, nmajor=bwd, out=self.q.get("w_" + which), **kw))
                self.q["w_" + which] = qw
            qw = self.q["w_" + which]
            self.out["y_" + which] = self._t(f"gemm_fwd_{which}", lambda: api.grouped_mm_fwd(
                qa, qw, self.ge, out=self.out.get("y_" + which)))
            if bwd:
                dy = data["dy_" + which]
                kw = dict(state=self.st_g, unit=gi) if r == "dl" else {}
                qd = self._t(f"quant_dy_{which}", lambda: api.quantize_act(
                    dy, r, self.fg, self.ge, rowwise=True, colwise=True, out=self.q.get("dy_" + which), **kw))
                self.q["dy_" + which] = qd
                self.out["da_" + which] = self._t(f"gemm_dgrad_{which}", lambda: api.grouped_mm_dgrad(
                    qd, qw, self.ge, out=self.out.get("da_" + which)))
                self.out["dw_" + which] = self._t(f"gemm_wgrad_{which}", lambda: api.grouped_mm_wgrad(
                    qa, qd, self.ge, out=self.out.get("dw_" + which), accumulate=not first))

    def work(self, R):
        """Algorithmic GEMM FLOPs and quantization bytes per call name."""
        spec, r = self.spec, self.recipe
        flops, byts = {}, {}
        per_layout = layout_bytes(r, self.fp4)
        read = 4.0 if r in ("tw", "nvfp4") else 2.0   # tw and nvfp4 read twice (tensor amax pass)
        w_layout = {"block": 1.0 + 4 / 16384}.get(r, per_layout)
        for which in spec.gemms:
            K, N = spec.gemm_shape(which)
            f = 2.0 * R * K * N
            flops[f"gemm_fwd_{which}"] = f
            nl = 2 if self.bwd else 1
            byts[f"quant_a_{which}"] = R * K * (read + nl * per_layout)
            byts[f"quant_w_{which}"] = self.E * K * N * (read + nl * w_layout)
            if self.bwd:
                flops[f"gemm_dgrad_{which}"] = f
                flops[f"gemm_wgrad_{which}"] = f
                byts[f"quant_dy_{which}"] = R * N * (read + 2 * per_layout)
        return flops, byts


def layout_bytes(recipe, fp4):
    """Algorithmic bytes per element of one quantized layout: the code plus
    its share of the scales (fp32 per 128 for blockwise, one E8M0 byte per
    32 for MX, one e4m3 byte per 16 for NVFP4)."""
    code = 0.5 if fp4 else 1.0
    return {"tw": code, "dl": code, "block": code + 4 / 128, "mx": code + 1 / 32,
            "nvfp4": code + 1 / 16}[recipe]


def gemm_peak(step):
    """(dense MFMA peak in TFLOP/s, the kernel's arithmetic) of the step's
    grouped GEMM."""
    if step.recipe == "nvfp4":
        return PEAK_F16_TFLOPS, "f16 MFMA over exactly dequantized NVFP4 operands"
    if step.fp4:
        return PEAK_FP4_TFLOPS, "fp4 scaled MFMA"
    return PEAK_FP8_TFLOPS, "fp8 scaled MFMA"


def attainable_ms(spec, group_sizes, modes, peak_tflops=PEAK_FP8_TFLOPS, code_bytes=1.0):
    """Roofline time of each GEMM call: sum over groups of max(FLOPs / MFMA
    peak, bytes / HBM peak), with a group's algorithmic bytes = its operand
    codes (code_bytes per element) read once plus its output written once
    (bf16 for forward and dgrad, fp32 dW for wgrad; an empty group still
    writes its zero dW)."""
    cb = code_bytes
    out = {}
    for which in spec.gemms:
        K, N = spec.gemm_shape(which)
        for mode in modes:
            t = 0.0
            for m in group_sizes:
                m = int(m)
                f = 2.0 * m * K * N
                if mode == "fwd":
                    b = (cb * (m * K + K * N) + 2 * m * N) if m else 0
                elif mode == "dgrad":
                    b = (cb * (m * N + K * N) + 2 * m * K) if m else 0
                else:
                    b = cb * (m * K + m * N) + 4 * K * N
                t = t + max(f / (peak_tflops * 1e12), b / (PEAK_HBM_GBS * 1e9))
            out[f"gemm_{mode}_{which}"] = t * 1e3
    return out


def swiglu_quant_rate(torch, api, step, spec, R):
    """The fused SwiGLU + quantization of the down-projection input, timed
    on its own after the step (the step's down-projection input is an input
    of the configuration): a random gate/up output [R, 2F] -> the step's
    layouts of silu(gate) * up [R, F]. None for workloads without a down
    projection."""
    if "dn" not in spec.gemms:
        return None
    F = spec.gemm_shape("dn")[0]
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    h = torch.randn(R, 2 * F, generator=g, device="cuda").to(torch.bfloat16)
    kw = {}
    if step.recipe == "dl":
        kw = dict(state=api.DelayedState.create(1, 0, 16), unit=0)
    q = api.quantize_act(h, step.recipe, step.fa, step.ge, rowwise=True, colwise=step.bwd,
                         swiglu=True, **kw)
    n = 10
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(n):
        api.quantize_act(h, step.recipe, step.fa, step.ge, rowwise=True, colwise=step.bwd,
                         swiglu=True, out=q, **kw)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    per_layout = layout_bytes(step.recipe, step.fp4)
    # gate and up (bf16); tensorwise and NVFP4 read them twice (amax pass)
    read = 8.0 if step.recipe in ("tw", "nvfp4") else 4.0
    nbytes = R * F * (read + (2 if step.bwd else 1) * per_layout)
    gbs = nbytes / (ms * 1e-3) / 1e9
    del h, q
    return {"rows": R, "F": F, "ms": round(ms, 4), "gbs": round(gbs, 1),
            "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}


def persistent_weights_rate(torch, step, sets, micro, step_flops, ms_step, quant_ms):
    """Optimizer steps of `micro` micro-batches with the weights quantized
    once per step (the persistent quantized weights of gradient
    accumulation), timed after the main loop: 1 untimed and 3 timed
    optimizer steps, micro-batches cycling through the input sets."""
    datas = [sets[i % len(sets)] for i in range(micro)]
    step.optimizer_step(datas)
    timing = []
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    n = 3
    torch.cuda.synchronize()
    e0.record()
    for _ in range(n):
        step.optimizer_step(datas, timing=timing)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    wq = sum(a.elapsed_time(b) for name, a, b in timing if name.startswith("quant_w")) / n
    wq_step = sum(v for k, v in quant_ms.items() if k.startswith("quant_w"))
    return {"micro_batches": micro, "ms_per_optimizer_step": round(ms, 4),
            "ms_per_micro_batch": round(ms / micro, 4),
            "tflops": round(step_flops * micro / (ms * 1e-3) / 1e12, 2),
            "weight_quant_ms_per_optimizer_step": round(wq, 4),
            "ms_per_step_weights_quantized_every_step": round(ms_step, 4),
            "weight_quant_ms_every_step": round(wq_step, 4),
            "note": "wgrad accumulates into fp32 after the first micro-batch; delayed update once per "
                    "optimizer step"}


def percentiles(v):
    """p10, median, p90 of a list of per-call times (ms)."""
    import numpy as np
    return [round(float(x), 4) for x in np.percentile(np.asarray(v, dtype=np.float64), [10, 50, 90])]


def cpu_baseline(cid, rows, cols, min_seconds=8.0):
    """The CPU oracle on a bounded sample of the same workload: the gate/up
    GEMM of the first experts that have routed rows, at most `rows` of each
    expert's rows, the full K and the first `cols` output columns, expert
    after expert until `min_seconds` of oracle work have been timed (one
    expert of the large configurations takes longer than that); quantization
    of the sampled operands plus the forward (and dgrad, wgrad) float64
    GEMMs. Reported in TFLOP/s of the sampled GEMMs."""
    import numpy as np
    from oracle import quant as OQ, gemm as OG, formats as OF
    from mx_scaled_grouped_amd import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    from oracle import routing as OR
    spec = W.SPECS[cid]
    topk = W.routing_for(cid)
    K, N = spec.gemm_shape("gu")
    N = min(N, cols)
    ends = OR.route(topk.expert_ids, topk.n_experts)["group_ends"].astype(np.int64)
    sizes = np.diff(np.concatenate([[0], ends]))
    experts = [int(e) for e in np.flatnonzero(sizes)]
    rec = {"tw": "tw", "dl": "dl", "block": "block", "mx": "mx", "mxfp4": "mx", "nvfp4": "nvfp4"}[spec.recipe]
    fq = OF.E2M1 if spec.recipe in ("mxfp4", "nvfp4") else OF.E4M3     # activations and weights
    bwd = "dgrad" in spec.modes
    fg = OF.E5M2 if rec == "dl" else fq
    dl = (np.float32(1.0), np.float32(1.0))

    def sc(q, key):
        return (q[key], q["tensor_scale"]) if rec == "nvfp4" else q[key]
    # synthetic operands of the sampled shapes (drawn once, outside the timing)
    mmax = min(rows, int(sizes.max()))
    a_all = W.normal_bf16(cid, W.T_X, (mmax, K))
    w = W.normal_bf16(cid, W.T_W1, (1, K, N), std=0.02, chunk_rows=256)
    dy_all = W.normal_bf16(cid, W.T_DY1, (mmax, N), std=2.0 ** -10) if bwd else None
    flops, dt, done, total_rows = 0.0, 0.0, [], 0
    for e in experts:
        m = min(rows, int(sizes[e]))
        a = a_all[:m]
        ge = np.array([m], np.int32)
        t0 = time.perf_counter()
        qa = OQ.quantize_act(a, rec, fq, ge, rowwise=True, colwise=bwd, dl_scale=dl)
        qw = OQ.quantize_weight(w, rec, fq, dl_scale=(np.ones(1, np.float32), np.ones(1, np.float32)))
        A = OG.deq_act_rows(qa["row_codes"], sc(qa, "row_scales"), rec, fq)
        OG.round_bf16(OG.grouped_fwd(A, OG.deq_weight(qw, rec, fq, "k"), ge))
        f = 2.0 * m * K * N
        if bwd:
            qd = OQ.quantize_act(dy_all[:m], rec, fg, ge, rowwise=True, colwise=True, dl_scale=dl)
            D = OG.deq_act_rows(qd["row_codes"], sc(qd, "row_scales"), rec, fg)
            OG.round_bf16(OG.grouped_dgrad(D, OG.deq_weight(qw, rec, fq, "n"), ge))
            P = qa["padded_starts"]
            At = OG.unpad_cols(OG.deq_act_cols(qa["col_codes"], sc(qa, "col_scales"), rec, fq), P, ge)
            Dt = OG.unpad_cols(OG.deq_act_cols(qd["col_codes"], sc(qd, "col_scales"), rec, fg), P, ge)
            OG.round_f32(OG.grouped_wgrad(At, Dt, ge, 1))
            f *= 3
        dt += time.perf_counter() - t0
        flops += f
        done.append(e)
        total_rows += m
        if dt >= min_seconds:
            break
    mode = "fwd+dgrad+wgrad" if bwd else "fwd"
    which = f"expert {done[0]}" if len(done) == 1 else f"experts {done[0]}-{done[-1]} ({len(done)})"
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{which} gate/up GEMM, {total_rows} routed rows (at most {rows} per expert, "
                      f"synthetic operands of those shapes) x K={K} x N={N}, {mode}, "
                      f"oracle quantization + float64 GEMMs, {dt:.1f} s"}


def cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or None."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def profile_values(workload):
    """Machine-read values of the committed counter summary of this
    workload's grouped GEMM: HBM bytes per launch (FETCH_SIZE and
    WRITE_SIZE, calibrated against a plain copy) and the time-weighted clock
    of the GEMM launches (GRBM_GUI_ACTIVE over kernel time). Empty when there
    is no summary or the GEMM source has changed since the counters were
    taken."""
    import hashlib
    path = os.path.join(HERE, "profiles", f"grouped_gemm_{workload}.md")
    if not os.path.exists(path):
        return {}
    kv = {}
    for line in open(path):
        if " = " in line:
            k, v = line.strip().split(" = ", 1)
            kv[k] = v
    src = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    if kv.get("gemm_source_sha256") != src:
        return {}
    out = {}
    if "traffic_bytes_per_launch" in kv:
        out["traffic"] = int(float(kv["traffic_bytes_per_launch"]))
    if "gemm_clock_ghz" in kv:
        out["clock_ghz"] = float(kv["gemm_clock_ghz"])
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); across GPUs the path "
              "would shard by expert, each GPU running this step on its own experts' groups",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from mx_scaled_grouped_amd import api, workloads as W

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}))
        return

    cid = WORKLOADS[args.workload]
    print(f"# generating inputs for {W.SPECS[cid].name}", file=sys.stderr, flush=True)
    spec, topk, ids, weights, sets = make_inputs(cid, torch, W, api)
    R = topk.rows
    step = Step(torch, api, spec, ids, weights, spec.recipe)
    group_sizes = torch.diff(step.ge.long(), prepend=step.ge.new_zeros(1).long()).cpu().numpy()
    torch.cuda.synchronize()
    print("# warmup", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step.run(sets[i % len(sets)])
    torch.cuda.synchronize()

    print("# timed steps", file=sys.stderr, flush=True)
    timing = []
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e_start.record()
    t_wall = time.perf_counter()
    for i in range(args.steps):
        step.run(sets[i % len(sets)], timing=timing)
    e_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_total = e_start.elapsed_time(e_end)
    ms_step = ms_total / args.steps

    per = {}
    for name, a, b in timing:
        per.setdefault(name, []).append(a.elapsed_time(b))
    flops, byts = step.work(R)
    step_flops = sum(flops.values())
    value = step_flops / (ms_step * 1e-3) / 1e12

    gemm_ms = {k: sum(v) / len(v) for k, v in per.items() if k.startswith("gemm")}
    quant_ms = {k: sum(v) / len(v) for k, v in per.items() if k.startswith("quant")}
    route_ms = sum(per["route"]) / len(per["route"])
    gemm_tflops = {k: flops[k] / (gemm_ms[k] * 1e-3) / 1e12 for k in gemm_ms}
    quant_gbs = {k: byts[k] / (quant_ms[k] * 1e-3) / 1e9 for k in quant_ms}
    gemm_total_ms = sum(gemm_ms.values())
    quant_total_ms = sum(quant_ms.values())
    # the dominant kernel is the grouped GEMM: every GEMM call is one launch of
    # it, so per-launch FLOPs / average launch time = step FLOPs / GEMM time
    launches = len(gemm_ms)
    achieved = step_flops / (gemm_total_ms * 1e-3) / 1e12
    quant_agg = sum(byts.values()) / (quant_total_ms * 1e-3) / 1e9
    peak, arith = gemm_peak(step)
    prof = profile_values(args.workload)
    att = attainable_ms(spec, group_sizes, spec.modes, peak, layout_bytes(step.recipe, step.fp4))
    att_frac = {k: att[k] / gemm_ms[k] for k in gemm_ms}
    att_total = sum(att[k] for k in gemm_ms) / gemm_total_ms

    # reference copy rates on the same GPU, 1 GiB device to device: the
    # library's streaming copy (16-byte streaming loads and stores, the
    # practical HBM ceiling the quantization passes are compared with next to
    # the 8 TB/s datasheet figure) and torch's own copy
    n_copy = 1 << 30
    src = torch.ones(n_copy, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)

    def copy_rate(fn):
        fn()
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        c0.record()
        for _ in range(5):
            fn()
        c1.record()
        torch.cuda.synchronize()
        return 2 * n_copy * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9

    # the engine clock under matrix-core load, right after the timed steps
    clock = api.clock_probe(iters=400000)
    copy_gbs = copy_rate(lambda: api.stream_copy(src, dst))
    torch_copy_gbs = copy_rate(lambda: dst.copy_(src))
    del src, dst
    swiglu = None if args.no_swiglu else swiglu_quant_rate(torch, api, step, spec, R)
    persistent = None
    if args.micro_batches > 1:
        persistent = persistent_weights_rate(torch, step, sets, args.micro_batches, step_flops, ms_step,
                                             quant_ms)

    cpu = None
    if not args.no_cpu_baseline:
        print("# cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(cid, args.cpu_sample_rows, args.cpu_sample_cols)

    out = {
        "metric": "FP8 grouped-GEMM TFLOP/s fwd+bwd (% FP8 MFMA peak); quant GB/s (% HBM)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"nvfp4": "fp4(e2m1) codes with e4m3 block scales and fp32 tensor scales",
                  "mx": "fp4(e2m1) codes with E8M0 block scales" if step.fp4 else "fp8(e4m3) codes with E8M0 block scales"
                  }.get(step.recipe, "fp8(e4m3/e5m2) codes")
                 + ", fp32 accumulate, bf16/fp32 out",
        "data": "synthetic (seeded torch generator on the GPU; routing seeded numpy)",
        "config": {"workload": spec.name, "experts": spec.experts, "tokens": spec.tokens,
                   "topk": spec.topk, "routed_rows": R, "hidden": spec.hidden, "ffn": spec.ffn,
                   "recipe": spec.recipe, "modes": list(spec.modes),
                   "group_sizes": [int(x) for x in group_sizes]},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": prof.get("traffic"),
                     "kernel": ("nvfp4_gemm_kernel" if step.recipe == "nvfp4" else "grouped_gemm_kernel")
                               + " (every GEMM launch of a step)",
                     "arithmetic": arith,
                     "launches_per_step": launches,
                     "flops_per_launch": step_flops / launches,
                     "avg_launch_ms": round(gemm_total_ms / launches, 4),
                     # the peak is quoted at 2.4 GHz. Two measured clocks: the clock probe's
                     # (bf16 MFMAs on every CU, run right after the timed steps) and the GEMM
                     # launches' own (PMC, from the committed profile of this source)
                     "sclk_mhz_measured": round(clock["mhz_median"], 1),
                     "sclk_source": "clock probe: bf16 MFMA load on every CU after the timed steps",
                     "peak_at_measured_sclk": round(peak * clock["mhz_median"] / 2400.0, 1),
                     "frac_at_measured_sclk": round(achieved / (peak * clock["mhz_median"] / 2400.0), 4),
                     "gemm_sclk_mhz_pmc": (round(prof["clock_ghz"] * 1000.0, 1) if "clock_ghz" in prof
                                           else None),
                     "frac_at_gemm_sclk_pmc": (round(achieved / (peak * prof["clock_ghz"] / 2.4), 4)
                                               if "clock_ghz" in prof else None)},
        "cpu_baseline": cpu,
        "breakdown": {
            "gemm_ms": {k: round(v, 4) for k, v in gemm_ms.items()},
            "gemm_tflops": {k: round(v, 1) for k, v in gemm_tflops.items()},
            "quant_ms": {k: round(v, 4) for k, v in quant_ms.items()},
            "quant_gbs": {k: round(v, 1) for k, v in quant_gbs.items()},
            "quant_gbs_total": round(quant_agg, 1),
            "quant_hbm_frac": round(quant_agg / PEAK_HBM_GBS, 4),
            "copy_1gib_gbs": round(copy_gbs, 1),
            "torch_copy_1gib_gbs": round(torch_copy_gbs, 1),
            "quant_copy_frac": round(quant_agg / copy_gbs, 4),
            "gemm_attainable_ms": {k: round(att[k], 4) for k in gemm_ms},
            "gemm_attainable_frac": {k: round(v, 4) for k, v in att_frac.items()},
            "gemm_attainable_frac_total": round(att_total, 4),
            "call_ms_p10_p50_p90": {k: percentiles(v) for k, v in per.items()},
            "route_ms": round(route_ms, 4),
            "gemm_ms_total": round(gemm_total_ms, 4),
            "quant_ms_total": round(quant_total_ms, 4),
            "wall_s": round(wall, 3),
            "swiglu_quant": swiglu,
            "clock_probe": clock,
            "persistent_weights": persistent,
        },
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
