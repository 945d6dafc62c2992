"""Helpers of the GPU parity tests: run the HIP path through the C ABI, run
the oracle on the same seeded inputs, and compare.

Routing is compared in three layers, because the GPU's fp32 logit sums are
rounded in a different order than the oracle's exact-then-rounded logits:
 1. select + routing_weights: the oracle's select and routing_weights applied
    to the GPU's own scores must reproduce the GPU's indices exactly and its
    weights within 1e-6 (this pins the selection logic bit for bit);
 2. scores: GPU scores are within a small relative distance of the oracle's;
 3. end to end: the GPU's indices equal the oracle's on every token, in
    order, and the per-expert counts equal the oracle's counts.  A token
    within tau = 8 x the largest selection-value difference of a tie has more
    than one correct top-k at the precision both sides decide in (f32); such
    a token may differ only if it is listed in NEAR_TIES with both candidate
    selections (recorded from a run, with its margin), and its pick must then
    still be a top-k of the oracle's own selection values up to tau.  Every
    case reports its smallest margin, tau and the number of tokens within tau.
Outputs: max |gpu - oracle| <= 2e-2 * rms(oracle) for bf16 outputs (the
bound the pages' measured drift supports), 1e-5 * rms + 1e-6 for f32.
"""

from __future__ import annotations

import math

import numpy as np
import torch

from mixture_experts_ffn_04_amd import api
from mixture_experts_ffn_04_amd import workloads as W
from oracle import moe_oracle as O

BF16_TOL = 2e-2        # max-abs error / rms(oracle output)

F32_TOL = 1e-5
WEIGHT_TOL = 1e-6

# Recorded near-ties: (workload name, T) -> {token: (oracle indices, GPU
# indices)}.  A token listed here sits within tau of a tie (its margin is
# recorded beside it); every other token of every case must match exactly.
NEAR_TIES: dict = {}


def host(t):
    return W.to_numpy_storage(t)


def sync():
    torch.cuda.synchronize()


class Case:
    """One workload: seeded inputs on the GPU, the HIP forward, oracle inputs."""

    def __init__(self, wl: W.Workload, device="cuda"):
        self.wl = wl
        self.cfg = api.config_from_workload(wl)
        self.device = device
        self.x = W.gen_x(wl, device)
        self.lw = api.layer_weights_from_workload(wl, device)
        self._experts = {}

    def forward(self, workspace=None):
        r = api.empty_routing(self.cfg, self.device)
        out = api.ffn_forward(self.cfg, self.x, self.lw, routing=r, workspace=workspace)
        sync()
        return out, r

    # ---------------- oracle side ----------------
    def x64(self):
        return O.to_f64(host(self.x), self.wl.act_dtype)

    def gate64(self):
        return O.to_f64(host(self.lw.gate_w), self.wl.act_dtype)

    def expert(self, e):
        if e not in self._experts:
            lw, wl = self.lw, self.wl
            if wl.w_dtype == "mxfp4":
                wgu = O.mxfp4_dequant(host(lw.w_gate_up[e]), host(lw.w_gate_up_scale[e]))
                wd = O.mxfp4_dequant(host(lw.w_down[e]), host(lw.w_down_scale[e]))
            else:
                wgu = O.to_f64(host(lw.w_gate_up[e]), wl.w_dtype)
                wd = O.to_f64(host(lw.w_down[e]), wl.w_dtype)
            bgu = O.to_f64(host(lw.b_gate_up[e]), wl.act_dtype) if lw.b_gate_up is not None else None
            bd = O.to_f64(host(lw.b_down[e]), wl.act_dtype) if lw.b_down is not None else None
            self._experts[e] = O.ExpertWeights(wgu, wd, bgu, bd)
        return self._experts[e]

    def shared64(self):
        lw, wl = self.lw, self.wl
        if lw.sh_gate_up is None:
            return None, None, None
        g = O.to_f64(host(lw.sh_gate), wl.act_dtype) if lw.sh_gate is not None else None
        return (O.to_f64(host(lw.sh_gate_up), wl.act_dtype), O.to_f64(host(lw.sh_down), wl.act_dtype), g)

    def bias(self, t):
        return None if t is None else host(t).astype(np.float32)

    def oracle_route(self):
        wl = self.wl
        return O.route(self.x64(), self.gate64(), k=wl.K, score_fn=wl.score_fn, n_group=wl.n_group,
                       topk_group=wl.topk_group, norm_topk_prob=wl.norm_topk_prob,
                       route_scale=wl.route_scale, expert_bias=self.bias(self.lw.expert_bias),
                       router_bias=self.bias(self.lw.router_bias))

    def oracle_forward(self):
        wl = self.wl
        shg, shd, shgate = self.shared64()
        return O.ffn_forward(self.x64(), self.gate64(), self.expert, n_experts=wl.E, k=wl.K,
                             score_fn=wl.score_fn, n_group=wl.n_group, topk_group=wl.topk_group,
                             norm_topk_prob=wl.norm_topk_prob, route_scale=wl.route_scale,
                             expert_bias=self.bias(self.lw.expert_bias),
                             router_bias=self.bias(self.lw.router_bias), limit=wl.swiglu_limit,
                             sh_gate_up64=shg, sh_down64=shd, sh_gate64=shgate, activation=wl.activation)

    def oracle_token(self, t, indices_row, weights_row):
        shg, shd, shgate = self.shared64()
        return O.token_output(self.x64()[t], indices_row, weights_row, self.expert,
                              self.wl.swiglu_limit, shg, shd, shgate, activation=self.wl.activation)


def check_routing(case: Case, o: O.RouteResult, g: api.Routing, report: dict):
    """Three-layer routing comparison (module docstring).  Returns (mask of
    tokens where the GPU picked differently inside a near-tie, the oracle's
    weights for the GPU's picks)."""
    wl = case.wl
    gs = g.scores.cpu().numpy()
    gi = g.indices.cpu().numpy()
    gw = g.weights.cpu().numpy()
    gc = g.counts.cpu().numpy()
    eb = case.bias(case.lw.expert_bias)

    # 1. selection logic, exactly, from the GPU's own scores
    gch = O.choice(gs, eb)
    sel = O.select(gch, wl.K, wl.n_group, wl.topk_group)
    assert np.array_equal(sel, gi), "select on the GPU scores differs from the GPU indices"
    w1 = O.routing_weights(gs, gi, wl.norm_topk_prob, wl.route_scale)
    report["weights_from_gpu_scores_maxabs"] = float(np.max(np.abs(w1 - gw))) if gw.size else 0.0
    assert report["weights_from_gpu_scores_maxabs"] <= WEIGHT_TOL

    # 2. scores
    ds = np.abs(gs.astype(np.float64) - o.scores.astype(np.float64))
    smax = float(np.max(np.abs(o.scores))) if o.scores.size else 1.0
    report["scores_maxabs"] = float(ds.max()) if ds.size else 0.0
    assert report["scores_maxabs"] <= 1e-5 * max(smax, 1e-30) + 1e-9

    # 3. end to end with the margin protocol
    dch = float(np.max(np.abs(gch.astype(np.float64) - o.choice.astype(np.float64)))) if gch.size else 0.0
    tau = 8.0 * max(dch, 1e-12)
    margins = O.selection_margins(o.choice, o.indices, wl.n_group, wl.topk_group)
    unique = margins > tau
    mism = np.any(gi != o.indices, axis=1)
    report.update(choice_maxabs=dch, tau=tau, min_margin=float(margins.min()) if margins.size else math.inf,
                  near_ties=int((~unique).sum()), index_mismatches=int(mism.sum()),
                  indices_equal_frac=float(1.0 - mism.mean()) if mism.size else 1.0)
    assert not np.any(mism & unique), "indices differ on a token with a clear margin"
    allowed = NEAR_TIES.get((wl.name, wl.T), {})
    expect = o.indices.copy()
    for t in np.nonzero(mism)[0]:
        assert int(t) in allowed, (f"token {t}: GPU picked {gi[t].tolist()}, oracle {o.indices[t].tolist()} "
                                   f"(margin {margins[t]:.3g}, tau {tau:.3g}); not a listed near-tie")
        want_oracle, want_gpu = allowed[int(t)]
        assert o.indices[t].tolist() == list(want_oracle) and gi[t].tolist() == list(want_gpu)
        assert valid_near_tie(o.choice[t], gi[t], tau, wl), f"token {t}: GPU pick is not a near-tie"
        expect[t] = gi[t]
    assert report["index_mismatches"] == len([t for t in allowed if t < len(mism)]), report
    assert np.array_equal(gc, O.expert_counts(expect, wl.E)), "per-expert counts differ from the oracle's"
    assert np.array_equal(gc, O.expert_counts(gi, wl.E)), "counts inconsistent with the GPU indices"
    # weights: the oracle's weights for the GPU's own selection
    ow = o.weights.copy()
    if mism.any():
        ow[mism] = O.routing_weights(o.scores[mism], gi[mism], wl.norm_topk_prob, wl.route_scale)
    dw = np.abs(gw - ow)
    report["weights_maxabs"] = float(dw.max()) if dw.size else 0.0
    assert report["weights_maxabs"] <= WEIGHT_TOL
    return mism, ow


def valid_near_tie(choice_row, picked, tau, wl):
    """The GPU's pick, measured by the oracle's selection values, is a top-K
    (and a top-topk_group group choice) up to tau, and is ordered up to tau."""
    c = np.asarray(choice_row, dtype=np.float64)
    picked = np.asarray(picked)
    allowed = np.ones(c.shape[0], dtype=bool)
    if wl.n_group > 1:
        gs = O.group_scores(choice_row, wl.n_group).astype(np.float64)
        size = c.shape[0] // wl.n_group
        kth = np.sort(gs)[::-1][wl.topk_group - 1]
        ok_groups = gs >= kth - 2 * tau
        used = np.unique(picked // size)
        if not np.all(ok_groups[used]) or len(used) > wl.topk_group:
            return False
        allowed = np.repeat(ok_groups, size)
    rest = np.ones(c.shape[0], dtype=bool)
    rest[picked] = False
    rest &= allowed
    if rest.any() and c[picked].min() < c[rest].max() - tau:
        return False
    return bool(np.all(c[picked][:-1] >= c[picked][1:] - tau))


def check_output(case: Case, gpu_out: torch.Tensor, ref: np.ndarray, report: dict, rows=None,
                 floor_allowance=0.0):
    """Max-abs error relative to the oracle output's RMS, with the bf16
    rounding floor reported beside it.  `floor_allowance` (used only for
    deliberately heavy-tailed outputs, where rounding the output to bf16 alone
    exceeds the bound) adds that many times the output's own bf16 rounding
    error to the bound."""
    got = gpu_out.float().cpu().numpy().astype(np.float64)
    if rows is not None:
        got = got[rows]
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    report.update(out_rms=rms, out_maxabs_err=err, out_err_over_rms=err / rms if rms else err)
    if case.wl.act_dtype == "bf16":
        floor = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()
        floor_abs = float(np.max(np.abs(floor - ref))) if ref.size else 0.0
        report["bf16_floor_over_rms"] = floor_abs / rms if rms else 0.0
        assert err <= BF16_TOL * rms + floor_allowance * floor_abs, report
    else:
        assert err <= F32_TOL * rms + 1e-6, report
    assert np.all(np.isfinite(got))
