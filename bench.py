#!/usr/bin/env python3
"""Throughput of the MoE FFN layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--T T]
                    [--score-fn FN] [--selection-bias] [--extra SPEC,...] [--no-extra]

One step = one moe_ffn_forward call (router, permutation, expert GEMMs, shared
expert, combine) on one batch of T tokens whose inputs already sit in HBM.
Expert weights rotate over several copies whose total exceeds the 256 MB
last-level cache when one copy fits in it, so every step reads its expert
weights from HBM (the DeepSeek-V4-style and qwen3_5_moe weights are 13 and 8
GB: one copy).

The headline is the largest workload that fits one GPU, the
DeepSeek-V4-style layer (E=256, I=2048, top-8 of 8 groups / 4, shared expert),
at T=72 (8 requests x verify block 9).  Extra lines: the same layer at
T=4096, and the other workloads at the token counts they are quoted on.

Prints ONE JSON line.  `value` is tokens/s of the whole layer, from a timed
loop of back-to-back forwards (`ms_per_step`); `ms_per_step_graph` replays the
same forwards captured in a HIP graph (four or more per graph).  `roofline` covers the dominant kernel
(routed gate_up + SwiGLU): algorithmic bytes (or flops) per launch divided by
its mean duration over a second timed loop of the same forwards, in which the
launch of that kernel carries HIP start/stop events that the GPU records at
the kernel's own start and end (hipExtLaunchKernelGGL on the launch stream).
`layer` gives the whole step against the layer's own roofline.  `traffic` is
the kernel's HBM bytes per launch from committed rocprofv3 counter runs,
reported only while the kernel sources still hash to the value recorded with
them.  `cpu_baseline` times the CPU oracle on a bounded sample of the
headline batch.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE FFN layer tokens/s at T=72 and T=4096; achieved HBM GB/s / MFMA % of peak"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
MALL_BYTES = 256 << 20
STAGE_GATE_UP, STAGE_DOWN = 3, 5

# workload specs: family[:T][:option]; options: sqrtsoftplus (score function),
# selbias (the qwen3_5_moe drafter with its bias as the selection-only expert bias),
# blockscaled (MXFP4 gate_up at large T on the block-scaled matrix cores)
HEADLINE = "deepseek_v4_style:72"
EXTRA = ("deepseek_v4_style:4096,qwen3_8b_moe_draft:72,qwen3_8b_moe_draft:8192,"
         "qwen3_5_moe_drafter:4096:selbias,qwen3_5_moe_drafter:4096,"
         "gpt_oss_style_mxfp4:72,gpt_oss_style_mxfp4:2048,gpt_oss_style_mxfp4:2048:blockscaled")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse_spec(spec):
    from mixture_experts_ffn_04_amd import workloads as W
    parts = spec.split(":")
    fam = parts[0]
    kw = {}
    if len(parts) > 1 and parts[1]:
        kw["T"] = int(parts[1])
    for opt in parts[2:]:
        if opt in ("sigmoid", "sqrtsoftplus"):
            kw["score_fn"] = opt
        elif opt == "selbias":
            kw["selection_bias"] = True
        elif opt == "blockscaled":
            kw["mx_gemm"] = "block_scaled"
        else:
            raise ValueError(f"unknown option {opt!r} in {spec!r}")
    if fam == "tiny_f32":
        return W.workload("tiny_f32")
    return W.workload(fam, **kw)


class HipEvents:
    """hipEvent_t handles for the library's measurement hook."""

    def __init__(self, n):
        self.rt = ctypes.CDLL("libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.start = (ctypes.c_void_p * n)()
        self.stop = (ctypes.c_void_p * n)()
        for arr in (self.start, self.stop):
            for i in range(n):
                h = ctypes.c_void_p()
                assert self.rt.hipEventCreate(ctypes.byref(h)) == 0
                arr[i] = h
        self.n = n

    def elapsed_ms(self):
        out = []
        for i in range(self.n):
            assert self.rt.hipEventSynchronize(self.stop[i]) == 0
            ms = ctypes.c_float()
            assert self.rt.hipEventElapsedTime(ctypes.byref(ms), self.start[i], self.stop[i]) == 0
            out.append(ms.value)
        return out

    def close(self):
        for arr in (self.start, self.stop):
            for i in range(self.n):
                self.rt.hipEventDestroy(arr[i])


def shared_in_routed(wl):
    """Whether the library runs the shared expert's gate_up items inside the
    routed gate_up launch: both on the streaming kernels (T below 256) with
    bf16 weights and activations."""
    return bool(wl.shared_I) and wl.T < 256 and wl.w_dtype == "bf16" and wl.act_dtype == "bf16"


def kernel_cost(wl, active, stage):
    """Algorithmic bytes and flops of one routed gate_up (or down) launch: the
    active experts' weights (+ MXFP4 scales, + linear biases) read once, the
    activation rows read (gate_up: x; down: h), the output written (gate_up:
    h in bf16; down: y in f32, or out in bf16 when each token has one expert
    and no shared expert); where the gate_up launch also runs the shared
    expert's items, its weights and its h."""
    H, I, K, T, Is = wl.H, wl.I, wl.K, wl.T, wl.shared_I
    act = 4 if wl.act_dtype == "f32" else 2
    sh = shared_in_routed(wl)
    if stage == "gate_up":
        if wl.w_dtype == "mxfp4":
            w = 2 * I * H // 2 + 2 * I * H // 32
        else:
            w = 2 * I * H * (4 if wl.w_dtype == "f32" else 2)
        b = 2 * I * act if wl.expert_linear_bias_std else 0
        byt = active * (w + b) + T * H * act + T * K * I * act
        flops = 4 * T * K * H * I
        if sh:
            byt += 2 * Is * H * act + T * Is * act
            flops += 4 * T * H * Is
        return byt, flops
    if wl.w_dtype == "mxfp4":
        w = H * I // 2 + H * I // 32
    else:
        w = H * I * (4 if wl.w_dtype == "f32" else 2)
    b = H * act if wl.expert_linear_bias_std else 0
    direct = K == 1 and not wl.shared_I
    out = T * H * act if direct else T * K * H * 4
    return active * (w + b) + T * K * I * act + out, 2 * T * K * H * I


def kernel_roofline(wl, active, stage, us):
    b, f = kernel_cost(wl, active, stage)
    t = us * 1e-6
    hbm_bound = b / (PEAK_HBM_GBS * 1e9) >= f / (PEAK_BF16_TFLOPS * 1e12)
    name = "routed gate_up + SwiGLU" if stage == "gate_up" else "routed down"
    if stage == "gate_up" and shared_in_routed(wl):
        name += " (with the shared expert's items)"
    if hbm_bound:
        ach = b / t / 1e9
        return {"kernel": name, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "kernel_us": round(us, 2),
                "algorithmic_bytes_per_launch": b}
    ach = f / t / 1e12
    return {"kernel": name, "bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "kernel_us": round(us, 2),
            "algorithmic_flops_per_launch": f}


def layer_roofline(wl, counts, ms):
    """The whole step against the layer's roofline: max(algorithmic bytes /
    8 TB/s, algorithmic flops / 2.5 PF/s)."""
    from mixture_experts_ffn_04_amd import workloads as W
    b = W.algorithmic_bytes(wl, counts)["total"]
    f = W.algorithmic_flops(wl)["total"]
    t_hbm = b / (PEAK_HBM_GBS * 1e9)
    t_mfma = f / (PEAK_BF16_TFLOPS * 1e12)
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    return {"bound": bound, "roofline_us": round(max(t_hbm, t_mfma) * 1e6, 1),
            "frac": round(max(t_hbm, t_mfma) / (ms * 1e-3), 4),
            "hbm_GBs": round(b / (ms * 1e-3) / 1e9, 1), "mfma_TFLOPs": round(f / (ms * 1e-3) / 1e12, 1),
            "algorithmic_bytes": b, "algorithmic_flops": f}


def stage_kernel_ms(L, cfg, x, sets, out, routing, ws, stage, steps):
    """Mean duration of the stage's kernel over `steps` forwards: the kernel's
    launch carries start/stop events that the GPU records at its own start
    and end."""
    import torch
    from mixture_experts_ffn_04_amd import _lib, api
    ev = HipEvents(steps)
    _lib.check(L.moe_profile_stage(stage, ev.start, ev.stop, steps))
    try:
        for i in range(steps):
            api.ffn_forward(cfg, x, sets[i % len(sets)], out=out, routing=routing, workspace=ws)
        torch.cuda.synchronize()
    finally:
        _lib.check(L.moe_profile_stage(-1, None, None, 0))
    ms = ev.elapsed_ms()
    ev.close()
    return sum(ms) / len(ms), min(ms), max(ms)


def run_gpu(wl, steps, warmup, copies=None, graph=True, min_warm_s=0.0):
    import torch
    from mixture_experts_ffn_04_amd import _lib, api
    from mixture_experts_ffn_04_amd import workloads as W

    dev = torch.device("cuda:0")
    cfg = api.config_from_workload(wl)
    log(f"workload {wl.name} T={wl.T}: drawing inputs")
    x = W.gen_x(wl, dev)
    base = api.layer_weights_from_workload(wl, dev)
    expert_bytes = sum(getattr(base, f).numel() * getattr(base, f).element_size()
                       for f in ("w_gate_up", "w_down", "w_gate_up_scale", "w_down_scale")
                       if getattr(base, f) is not None)
    if copies is None:
        copies = 1 if expert_bytes > 4 * MALL_BYTES else max(2, math.ceil(1.2e9 / expert_bytes))
        copies = min(copies, 8)
    sets = [base]
    for _ in range(copies - 1):
        kw = {f: getattr(base, f) for f in api.LayerWeights.FIELDS}
        for f in ("w_gate_up", "w_down", "w_gate_up_scale", "w_down_scale"):
            if kw[f] is not None:
                kw[f] = kw[f].clone()
        sets.append(api.LayerWeights(**kw))
    ws = api.alloc_workspace(cfg, dev)
    out = torch.empty(wl.T, wl.H, dtype=wl.torch_act_dtype, device=dev)
    routing = api.empty_routing(cfg, dev)
    log(f"expert weights {expert_bytes / 1e6:.1f} MB x {copies} copies; warmup {warmup}")
    t_warm = time.perf_counter()
    for i in range(warmup):
        api.ffn_forward(cfg, x, sets[i % copies], out=out, routing=routing, workspace=ws)
    torch.cuda.synchronize()
    # extra lines: more untimed forwards until the GPU has run for min_warm_s
    # (after the host-side input generation its clock needs a moment to rise)
    i = warmup
    while time.perf_counter() - t_warm < min_warm_s:
        api.ffn_forward(cfg, x, sets[i % copies], out=out, routing=routing, workspace=ws)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

    # timed loop: the layer alone, back to back
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        api.ffn_forward(cfg, x, sets[i % copies], out=out, routing=routing, workspace=ws)
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)

    # the same forwards replayed from a HIP graph: at least four captured
    # forwards per graph (cycling over the weight copies), as a serving graph
    # holds many layers, so one graph launch is not charged to a single layer
    graph_ms = None
    if graph:
        per_graph = max(copies, 4)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in range(per_graph):
                api.ffn_forward(cfg, x, sets[i % copies], out=out, routing=routing, workspace=ws)
        reps = max(1, steps // per_graph)
        g.replay()
        torch.cuda.synchronize()
        t0.record()
        for _ in range(reps):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        graph_ms = t0.elapsed_time(t1) / (reps * per_graph)
        del g

    L = _lib.lib()
    gu = stage_kernel_ms(L, cfg, x, sets, out, routing, ws, STAGE_GATE_UP, steps)
    dn = stage_kernel_ms(L, cfg, x, sets, out, routing, ws, STAGE_DOWN, steps)
    counts = routing.counts.cpu().numpy()
    active = int((counts > 0).sum())
    log(f"timed {steps} steps: {total_ms / steps * 1e3:.1f} us/step"
        + (f", graph {graph_ms * 1e3:.1f} us/step" if graph_ms else "")
        + f", gate_up {gu[0] * 1e3:.1f} us, down {dn[0] * 1e3:.1f} us, active experts {active}")
    res = dict(ms_per_step=total_ms / steps, graph_ms=graph_ms, gate_up_ms=gu, down_ms=dn, active=active,
               counts=counts, max_count=int(counts.max()), copies=copies, expert_bytes=expert_bytes)
    host = dict(x=x, base=base, routing=routing)
    return res, host


def time_backward(wl, host, steps):
    """Per-call time of the layer's backward (moe_ffn_backward) on this
    batch, against its own roofline: the larger of the HBM floor (expert
    weights read, gate_up twice and down once, for the active experts; every
    expert's f32 weight gradient written, experts without rows get zeros;
    x and dout read, dx written) and the matrix-core floor.  The backward's
    products run on bf16 MFMA with f32 accumulation; an f32 or scaled operand
    enters as an exact bf16 hi/lo pair, so a product whose two operands are
    both split takes three MFMA passes (hi*hi + lo*hi + hi*lo) and one with
    a single split operand takes two.  The matrix-core floor prices the
    passes the kernels execute at the bf16 peak; the algorithmic flop count
    (2 x 9 T K H I routed + 2 x 9 T H Is shared + 2 x 2 T E H router) and
    its rate are reported beside it.  The backward is for training; the
    serving step above does not include it."""
    import torch
    from mixture_experts_ffn_04_amd import api
    from mixture_experts_ffn_04_amd import workloads as W

    if wl.w_dtype == "mxfp4":
        return None
    cfg = api.config_from_workload(wl)
    x, lw, r = host["x"], host["base"], host["routing"]
    dout = W.gen_dout(wl, x.device)
    ws = torch.empty(max(api.backward_workspace_bytes(cfg), 256), dtype=torch.uint8, device=x.device)
    for _ in range(2):
        api.ffn_backward(cfg, x, lw, dout, r, workspace=ws)
    n = max(3, steps // 20)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(n):
        api.ffn_backward(cfg, x, lw, dout, r, workspace=ws)
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) / n * 1e3
    active = int((r.counts > 0).sum().item())
    wb = 2 if wl.w_dtype == "bf16" else 4
    ab = 2 if wl.act_dtype == "bf16" else 4
    per_expert = wl.H * wl.I
    weight_reads = active * (2 * 2 * per_expert + per_expert) * wb
    grad_writes = wl.E * 3 * per_expert * 4 + wl.E * wl.H * 4
    if wl.shared_I:
        weight_reads += 3 * wl.H * wl.shared_I * ab
        grad_writes += 3 * wl.H * wl.shared_I * 4
    act = wl.T * wl.H * (2 * ab + 4) + wl.T * wl.E * 4
    nbytes = weight_reads + grad_writes + act
    flops = 18 * wl.T * wl.K * wl.H * wl.I + 18 * wl.T * wl.H * wl.shared_I + 4 * wl.T * wl.E * wl.H
    # executed bf16 MFMA flops: passes = 1 + (A split) + (B split)
    xs = 0 if wl.act_dtype == "bf16" else 1      # x, dout, shared weights
    ws_ = 0 if wl.w_dtype == "bf16" else 1       # routed expert weights
    R, H, I, Is, T, E = wl.T * wl.K, wl.H, wl.I, wl.shared_I, wl.T, wl.E
    routed = (2 * R * H * 2 * I * (1 + xs + ws_)      # pre = x_rows Wgu^T
              + 2 * R * H * I * (1 + xs + ws_)        # gd = dout_rows Wd
              + 2 * R * 2 * I * H * (2 + ws_)         # dx_rows = dpre Wgu (dpre f32)
              + 2 * R * H * I * 3                     # dWd: (w dout)^T h, both split
              + 2 * R * 2 * I * H * (2 + xs))         # dWgu: dpre^T x
    gated = 1 if wl.shared_gated else 0
    shared = 0
    if Is:
        shared = (2 * T * H * 2 * Is * (1 + 2 * xs) + 2 * T * H * Is * (1 + 2 * xs)
                  + 2 * T * 2 * Is * H * (2 + xs) + 2 * T * H * Is * (2 + max(xs, gated))
                  + 2 * T * 2 * Is * H * (2 + xs))
    router = 2 * E * T * H * (2 + xs) * 2
    mfma_flops = routed + shared + router
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    t_mfma = mfma_flops / (PEAK_BF16_TFLOPS * 1e12)
    floor = max(t_hbm, t_mfma)
    return {"us": round(us, 2), "bound": "hbm" if t_hbm >= t_mfma else "mfma",
            "floor_us": round(floor * 1e6, 1), "frac": round(floor / (us * 1e-6), 4),
            "algorithmic_bytes": nbytes, "algorithmic_flops": flops, "mfma_pass_flops": mfma_flops,
            "hbm_GBs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "mfma_TFLOPs": round(mfma_flops / (us * 1e-6) / 1e12, 2),
            "algorithmic_TFLOPs": round(flops / (us * 1e-6) / 1e12, 2)}


def time_balance(wl, routing, steps):
    """Per-call time of the load-balancing state on this batch's routing: the
    masked kept-slot count (one per forward) and the step balance + bias sign
    step + reset (one per optimizer step)."""
    import torch
    from mixture_experts_ffn_04_amd import api
    from mixture_experts_ffn_04_amd import workloads as W

    dev = routing.indices.device
    _, mask, bias = W.gen_balance_inputs(0, wl.T, wl.K, wl.E, keep=0.8)
    mask, bias = mask.to(dev), bias.to(dev)
    counts = torch.zeros(wl.E, dtype=torch.int64, device=dev)
    sb = torch.empty(1, dtype=torch.float32, device=dev)
    for _ in range(3):
        api.balance_count(routing.indices, counts, mask)
        api.balance_update(counts, bias, 1e-3, sb)
    t = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    torch.cuda.synchronize()
    t[0].record()
    for _ in range(steps):
        api.balance_count(routing.indices, counts, mask)
    t[1].record()
    for _ in range(steps):
        api.balance_update(counts, bias, 1e-3, sb)
    t[2].record()
    torch.cuda.synchronize()
    return {"count_us": round(t[0].elapsed_time(t[1]) / steps * 1e3, 2),
            "update_us": round(t[1].elapsed_time(t[2]) / steps * 1e3, 2),
            "slots": wl.T * wl.K, "experts": wl.E}


# HBM traffic of the dominant kernel, per launch, from rocprofv3 FETCH_SIZE /
# WRITE_SIZE counter runs (scaled by a plain copy of known size), with the
# hash of the kernel sources they were taken on: a changed kernel reports null.
TRAFFIC_RECORDS = {
    ("deepseek_v4_style_e256_top8_sigmoid", 72): "profiles/stream_gate_up_deepseek_v4_style_t72_pmc.md",
    ("qwen3_8b_moe_draft_e8_top1", 72): "profiles/stream_gate_up_qwen3_8b_moe_draft_t72_pmc.md",
}
KERNEL_SOURCES = ["mixture_experts_ffn_04_amd/csrc/stream.hip", "mixture_experts_ffn_04_amd/csrc/common.hpp",
                  "mixture_experts_ffn_04_amd/csrc/tile.hpp"]


def kernel_sources_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(wl):
    path = TRAFFIC_RECORDS.get((wl.name, wl.T))
    if not path or not os.path.exists(os.path.join(ROOT, path)):
        return None
    fields = {}
    with open(os.path.join(ROOT, path)) as fh:
        for ln in fh:
            if ":" in ln and ln.strip().startswith(("traffic_", "kernel_sources_sha256")):
                k, v = ln.strip().split(":", 1)
                fields[k.strip()] = v.strip().replace(",", "")
    if fields.get("kernel_sources_sha256") != kernel_sources_hash():
        return None
    try:
        return int(fields["traffic_fetch_bytes_per_launch"]) + int(fields["traffic_write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def line_for(wl, res):
    """Throughput, graph replay, kernel and layer rooflines of one run."""
    gu_ms, dn_ms = res["gate_up_ms"], res["down_ms"]
    roof = kernel_roofline(wl, res["active"], "gate_up", gu_ms[0] * 1e3)
    roof["traffic"] = recorded_traffic(wl) if roof["bound"] == "hbm" else None
    roof["kernel_us_min_max"] = [round(gu_ms[1] * 1e3, 2), round(gu_ms[2] * 1e3, 2)]
    down = kernel_roofline(wl, res["active"], "down", dn_ms[0] * 1e3)
    return {
        "value": round(wl.T / (res["ms_per_step"] * 1e-3), 1),
        "ms_per_step": round(res["ms_per_step"], 5),
        "ms_per_step_graph": round(res["graph_ms"], 5) if res["graph_ms"] else None,
        "roofline": roof,
        "down": down,
        "layer": layer_roofline(wl, res["counts"], res["ms_per_step"]),
    }


def workload_config(wl, res):
    cfg = {"workload": wl.name, "T": wl.T, "H": wl.H, "E": wl.E, "I": wl.I, "K": wl.K,
           "score_fn": wl.score_fn, "expert_weights": wl.w_dtype, "weight_copies": res["copies"],
           "active_experts": res["active"], "max_tokens_per_expert": res["max_count"]}
    if wl.n_group > 1:
        cfg["groups"] = [wl.n_group, wl.topk_group]
    if wl.shared_I:
        cfg["shared_I"] = wl.shared_I
    if wl.expert_bias_std:
        cfg["expert_bias_std"] = wl.expert_bias_std
    if wl.router_bias_std:
        cfg["router_bias_std"] = wl.router_bias_std
    if res["copies"] == 1 and res["expert_bytes"] <= MALL_BYTES:
        cfg["weights_cache"] = "warm (one copy fits the 256 MB last-level cache)"
    return cfg


def host_info():
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"host_cpus": os.cpu_count(), "cpu_model": model}


def cpu_baseline(wl, host, budget_s):
    """The oracle, as it stands, on a bounded sample of the same batch: its
    first tokens, one oracle call per token (a token's output does not depend
    on the other tokens of the batch), until the time budget is spent.  The
    weights of the experts those tokens use are copied to the host first
    (outside the timed region); the oracle widens them to fp64 per call."""
    import numpy as np
    from mixture_experts_ffn_04_amd import workloads as W
    from oracle import moe_oracle as O

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    base = host["base"]
    st = W.to_numpy_storage
    x_h = st(host["x"])
    gate_h = st(base.gate_w)
    eb = st(base.expert_bias) if base.expert_bias is not None else None
    rb = st(base.router_bias) if base.router_bias is not None else None
    gi = host["routing"].indices.cpu().numpy()
    store = {}

    def fetch(e):
        if e not in store:
            if wl.w_dtype == "mxfp4":
                store[e] = (st(base.w_gate_up[e]), st(base.w_gate_up_scale[e]), st(base.w_down[e]),
                            st(base.w_down_scale[e]))
            else:
                store[e] = (st(base.w_gate_up[e]), st(base.w_down[e]))
        return store[e]

    bgu = st(base.b_gate_up) if base.b_gate_up is not None else None
    bd = st(base.b_down) if base.b_down is not None else None
    sh = (st(base.sh_gate_up), st(base.sh_down)) if base.sh_gate_up is not None else None
    shg = st(base.sh_gate) if base.sh_gate is not None else None
    ad = wl.act_dtype

    def get_expert(e):
        s = fetch(e)
        if wl.w_dtype == "mxfp4":
            wgu, wd = O.mxfp4_dequant(s[0], s[1]), O.mxfp4_dequant(s[2], s[3])
        else:
            wgu, wd = O.to_f64(s[0], wl.w_dtype), O.to_f64(s[1], wl.w_dtype)
        return O.ExpertWeights(wgu, wd, O.to_f64(bgu[e], ad) if bgu is not None else None,
                               O.to_f64(bd[e], ad) if bd is not None else None)

    def once(t0, t1):
        return O.ffn_forward(
            O.to_f64(x_h[t0:t1], ad), O.to_f64(gate_h, ad), get_expert, n_experts=wl.E, k=wl.K,
            score_fn=wl.score_fn, n_group=wl.n_group, topk_group=wl.topk_group,
            norm_topk_prob=wl.norm_topk_prob, route_scale=wl.route_scale,
            expert_bias=eb, router_bias=rb, limit=wl.swiglu_limit, activation=wl.activation,
            sh_gate_up64=O.to_f64(sh[0], ad) if sh else None,
            sh_down64=O.to_f64(sh[1], ad) if sh else None,
            sh_gate64=O.to_f64(shg, ad) if shg is not None else None)

    tokens, t_total = 0, 0.0
    while tokens < wl.T and (tokens < 1 or t_total < budget_s):
        for e in gi[tokens].tolist():      # host copies outside the timed region
            fetch(e)
        t = time.perf_counter()
        once(tokens, tokens + 1)
        t_total += time.perf_counter() - t
        tokens += 1
    return {"value": round(tokens / t_total, 3), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"first {tokens} of the T={wl.T} batch of {wl.name}, one token per oracle call, "
                      f"{t_total:.1f} s (numpy fp64 oracle incl. widening the bf16/MXFP4 weights; "
                      f"cores = BLAS threads it ran with)",
            **host_info()}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, help="family (default: the headline, " + HEADLINE + ")")
    ap.add_argument("--T", type=int, default=None)
    ap.add_argument("--score-fn", default=None)
    ap.add_argument("--selection-bias", action="store_true")
    ap.add_argument("--mx-block-scaled", action="store_true",
                    help="MXFP4 gate_up at large T on the block-scaled matrix cores")
    ap.add_argument("--copies", type=int, default=None)
    ap.add_argument("--extra", default=EXTRA, help="comma-separated family:T[:option] specs")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run device-to-device copies of MIB MiB (the reference kernel "
                         "for scaling FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the library has no "
              "multi-GPU path)", file=sys.stderr)
        return 2

    if args.copy_calibration:
        import torch
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 5}), flush=True)
        return 0

    if args.workload is None:
        wl = parse_spec(HEADLINE)
    else:
        spec = args.workload + (f":{args.T}" if args.T else ":")
        if args.score_fn:
            spec += f":{args.score_fn}"
        if args.selection_bias:
            spec += ":selbias"
        if args.mx_block_scaled:
            spec += ":blockscaled"
        wl = parse_spec(spec)
    if args.T and args.workload is None:
        wl = wl.with_T(args.T)

    import torch
    res, host = run_gpu(wl, args.steps, args.warmup, args.copies, graph=not args.no_graph)
    main_line = line_for(wl, res)
    line = {
        "metric": METRIC, "value": main_line["value"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": main_line["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if wl.act_dtype == "bf16" else "f32", "data": "synthetic",
        "config": workload_config(wl, res),
        "ms_per_step_graph": main_line["ms_per_step_graph"],
        "roofline": main_line["roofline"],
        "down": main_line["down"],
        "layer": main_line["layer"],
        "balance": time_balance(wl, host["routing"], args.steps),
    }
    if not args.no_backward:
        line["backward"] = time_backward(wl, host, args.steps)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        line["cpu_baseline"] = cpu_baseline(wl, host, args.cpu_seconds)
    del host
    torch.cuda.empty_cache()

    extra = []
    if not args.no_extra and args.extra:
        for spec in args.extra.split(","):
            wl2 = parse_spec(spec)
            if (wl2.name, wl2.T) == (wl.name, wl.T):
                continue
            large = wl2.T >= 1024
            res2, host2 = run_gpu(wl2, max(10, args.steps // 2) if large else args.steps,
                                  max(2, args.warmup // 2) if large else args.warmup,
                                  graph=not args.no_graph, min_warm_s=0.3)
            e = line_for(wl2, res2)
            extra.append({"workload": wl2.name, "T": wl2.T, "unit": "tokens/s",
                          "config": workload_config(wl2, res2), **e})
            del host2, res2
            torch.cuda.empty_cache()
    if extra:
        line["extra"] = extra
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
