#!/usr/bin/env python3
"""Throughput of the MoE FFN layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--T T]

One step = one moe_ffn_forward call (router, permutation, expert GEMMs,
combine, shared expert) on one batch of T tokens whose inputs already sit in
HBM.  Expert weights rotate over several copies whose total exceeds the
256 MB last-level cache, so every step reads its expert weights from HBM.

Prints ONE JSON line.  `value` is tokens/s of the whole layer, from a timed
loop of back-to-back forwards.  `roofline` covers the dominant kernel (routed
gate_up + SwiGLU): algorithmic bytes (or flops) per launch divided by its mean
duration, timed with HIP events recorded on the launch stream around that
kernel in a second timed loop of the same forwards.
The bracketed durations include the cost of an event pair, which is
measured on the same stream with nothing between the events and subtracted
(both numbers are reported).  `traffic` is the kernel's HBM bytes per launch
from committed rocprofv3 counter runs, reported only while the kernel sources
still hash to the value recorded with them.
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE FFN layer tokens/s at T=72 and T=4096; achieved HBM GB/s / MFMA % of peak"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
MALL_BYTES = 256 << 20
STAGE_GATE_UP = 3


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles for the library's measurement hook."""

    def __init__(self, n):
        self.rt = ctypes.CDLL("libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
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


def gate_up_cost(wl, active, T):
    """Algorithmic bytes and flops of one routed gate_up launch: the active
    experts' gate/up weights (+ MXFP4 scales, + linear biases) read once, the
    activation rows read, the SwiGLU output h written."""
    H, I, K = wl.H, wl.I, wl.K
    if wl.w_dtype == "mxfp4":
        w = 2 * I * H // 2 + 2 * I * H // 32
    else:
        w = 2 * I * H * (4 if wl.w_dtype == "f32" else 2)
    act = 4 if wl.act_dtype == "f32" else 2
    b = 2 * I * act if wl.expert_linear_bias_std else 0
    bytes_ = active * (w + b) + T * H * act + T * K * I * act
    flops = 4 * T * K * H * I
    return bytes_, flops


def run_gpu(wl, steps, warmup, copies=None):
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
    for i in range(warmup):
        api.ffn_forward(cfg, x, sets[i % copies], out=out, routing=routing, workspace=ws)
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
    # second timed loop with HIP events recorded on the launch stream around
    # the routed gate_up kernel(s) (the events add idle gaps, so this loop
    # does not feed `value`)
    ev = HipEvents(steps)
    L = _lib.lib()
    _lib.check(L.moe_profile_stage(STAGE_GATE_UP, ev.start, ev.stop, steps))
    for i in range(steps):
        api.ffn_forward(cfg, x, sets[i % copies], out=out, routing=routing, workspace=ws)
    torch.cuda.synchronize()
    _lib.check(L.moe_profile_stage(-1, None, None, 0))
    k_ms = ev.elapsed_ms()
    # cost of an event pair with nothing between it, on the same stream: the
    # bracketed durations above include it, the kernel's own duration does not
    stream = torch.cuda.current_stream().cuda_stream
    for i in range(steps):
        assert ev.rt.hipEventRecord(ev.start[i], ctypes.c_void_p(stream)) == 0
        assert ev.rt.hipEventRecord(ev.stop[i], ctypes.c_void_p(stream)) == 0
    torch.cuda.synchronize()
    pair_ms = ev.elapsed_ms()
    ev.close()
    counts = routing.counts.cpu().numpy()
    active = int((counts > 0).sum())
    log(f"timed {steps} steps: {total_ms / steps * 1e3:.1f} us/step, gate_up "
        f"{sum(k_ms) / len(k_ms) * 1e3:.1f} us, active experts {active}")
    event_ms = sum(k_ms) / len(k_ms)
    pair = sum(pair_ms) / len(pair_ms)
    res = dict(ms_per_step=total_ms / steps, kernel_ms=max(event_ms - pair, 1e-6), event_ms=event_ms,
               pair_ms=pair, active=active,
               max_count=int(counts.max()), copies=copies, expert_bytes=expert_bytes)
    host = dict(x=x, base=base, routing=routing)
    return res, host


def time_backward(wl, host, steps):
    """Per-call time of the layer's backward (moe_ffn_backward) on this
    batch, with the HBM floor it is measured against: expert weights read
    (active experts; gate_up twice, down once), every expert's f32 weight
    gradient written (experts without rows get zeros), x, dout read and dx
    written.  The backward is for training; the serving step above does not
    include it."""
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
    return {"us": round(us, 2), "bound": "hbm", "algorithmic_bytes": nbytes,
            "achieved": round(nbytes / (us * 1e-6) / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}


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
    ("qwen3_8b_moe_draft_e8_top1", 72): "profiles/stream_gate_up_qwen3_8b_moe_draft_t72_pmc.md",
}
KERNEL_SOURCES = ["mixture_experts_ffn_04_amd/csrc/stream.hip", "mixture_experts_ffn_04_amd/csrc/common.hpp",
                  "mixture_experts_ffn_04_amd/csrc/tile.hpp"]


def kernel_sources_hash():
    import hashlib
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


def roofline(wl, res):
    b, f = gate_up_cost(wl, res["active"], wl.T)
    t = res["kernel_ms"] * 1e-3
    hbm_bound = b / (PEAK_HBM_GBS * 1e9) >= f / (PEAK_BF16_TFLOPS * 1e12)
    timing = {"kernel_us": round(res["kernel_ms"] * 1e3, 2), "event_bracket_us": round(res["event_ms"] * 1e3, 2),
              "empty_event_pair_us": round(res["pair_ms"] * 1e3, 2)}
    if hbm_bound:
        ach = b / t / 1e9
        return {"kernel": "routed gate_up + SwiGLU", "bound": "hbm", "achieved": round(ach, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                "traffic": recorded_traffic(wl), "algorithmic_bytes_per_launch": b, **timing}
    ach = f / t / 1e12
    return {"kernel": "routed gate_up + SwiGLU", "bound": "mfma", "achieved": round(ach, 1),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
            "traffic": None, "algorithmic_flops_per_launch": f, **timing}


def cpu_baseline(wl, host, budget_s):
    """The oracle, as it stands, on the same inputs (copied to the host), over
    a bounded number of whole-batch repetitions."""
    import numpy as np
    from mixture_experts_ffn_04_amd import workloads as W
    from oracle import moe_oracle as O

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    base = host["base"]
    st = W.to_numpy_storage
    x_h = st(host["x"])
    gate_h = st(base.gate_w)
    eb = st(base.expert_bias) if base.expert_bias is not None else None
    rb = st(base.router_bias) if base.router_bias is not None else None
    # expert weights of the experts this batch uses, in storage format
    used = sorted(set(host["routing"].indices.cpu().numpy().ravel().tolist()))
    store = {}
    for e in used:
        if wl.w_dtype == "mxfp4":
            store[e] = (st(base.w_gate_up[e]), st(base.w_gate_up_scale[e]), st(base.w_down[e]),
                        st(base.w_down_scale[e]))
        else:
            store[e] = (st(base.w_gate_up[e]), st(base.w_down[e]))
    bgu = {e: st(base.b_gate_up[e]) for e in used} if base.b_gate_up is not None else None
    bd = {e: st(base.b_down[e]) for e in used} if base.b_down is not None else None
    sh = (st(base.sh_gate_up), st(base.sh_down)) if base.sh_gate_up is not None else None
    shg = st(base.sh_gate) if base.sh_gate is not None else None
    ad = wl.act_dtype

    def get_expert(e):
        s = store[e]
        if wl.w_dtype == "mxfp4":
            wgu, wd = O.mxfp4_dequant(s[0], s[1]), O.mxfp4_dequant(s[2], s[3])
        else:
            wgu, wd = O.to_f64(s[0], wl.w_dtype), O.to_f64(s[1], wl.w_dtype)
        return O.ExpertWeights(wgu, wd, O.to_f64(bgu[e], ad) if bgu else None,
                               O.to_f64(bd[e], ad) if bd else None)

    def once():
        return O.ffn_forward(
            O.to_f64(x_h, ad), O.to_f64(gate_h, ad), get_expert, n_experts=wl.E, k=wl.K,
            score_fn=wl.score_fn, n_group=wl.n_group, topk_group=wl.topk_group,
            norm_topk_prob=wl.norm_topk_prob, route_scale=wl.route_scale,
            expert_bias=eb, router_bias=rb, limit=wl.swiglu_limit,
            sh_gate_up64=O.to_f64(sh[0], ad) if sh else None,
            sh_down64=O.to_f64(sh[1], ad) if sh else None,
            sh_gate64=O.to_f64(shg, ad) if shg is not None else None)

    reps, t_total = 0, 0.0
    while reps < 1 or (t_total < budget_s and reps < 500):
        t = time.perf_counter()
        once()
        t_total += time.perf_counter() - t
        reps += 1
    return {"value": round(reps * wl.T / t_total, 2), "unit": "tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{reps} whole-batch forward(s) of T={wl.T} ({wl.name}), "
                      f"{t_total:.1f} s, numpy fp64 oracle incl. weight decoding"}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="qwen3_8b_moe_draft")
    ap.add_argument("--T", type=int, default=72)
    ap.add_argument("--score-fn", default=None)
    ap.add_argument("--copies", type=int, default=None)
    ap.add_argument("--extra-T", type=int, default=8192,
                    help="also time the same family at this token count (0 = skip)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run device-to-device copies of MIB MiB (the reference kernel "
                         "for scaling FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args(argv)

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

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the library has no "
              "multi-GPU path)", file=sys.stderr)
        return 2

    from mixture_experts_ffn_04_amd import workloads as W
    kw = {"T": args.T}
    if args.score_fn:
        kw["score_fn"] = args.score_fn
    wl = W.workload(args.workload, **kw) if args.workload != "tiny_f32" else W.workload("tiny_f32")

    res, host = run_gpu(wl, args.steps, args.warmup, args.copies)
    value = wl.T / (res["ms_per_step"] * 1e-3)
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(res["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if wl.act_dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "H": wl.H, "E": wl.E, "I": wl.I, "K": wl.K,
                   "expert_weights": wl.w_dtype, "weight_copies": res["copies"],
                   "active_experts": res["active"], "max_tokens_per_expert": res["max_count"]},
        "roofline": roofline(wl, res),
        "balance": time_balance(wl, host["routing"], args.steps),
        "backward": time_backward(wl, host, args.steps),
    }
    extra = []
    if args.extra_T and args.extra_T != wl.T and args.workload != "tiny_f32":
        import torch
        del host
        torch.cuda.empty_cache()
        wl2 = wl.with_T(args.extra_T)
        res2, host2 = run_gpu(wl2, max(10, args.steps // 10), max(3, args.warmup // 4), copies=1)
        extra.append({"workload": wl2.name, "T": wl2.T,
                      "value": round(wl2.T / (res2["ms_per_step"] * 1e-3), 1), "unit": "tokens/s",
                      "ms_per_step": round(res2["ms_per_step"], 5), "roofline": roofline(wl2, res2)})
        del host2
        torch.cuda.empty_cache()
        _, host = run_gpu(wl, 2, 1, copies=1)  # inputs of the headline batch for the CPU leg
    if extra:
        line["extra"] = extra
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        line["cpu_baseline"] = cpu_baseline(wl, host, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
