"""Torch-tensor front end of the C ABI (argument marshalling only).

Every step of the layer runs in libmoe_ffn.so; this module checks shapes,
dtypes, devices and contiguity, allocates outputs and the workspace with
torch (device memory only), and passes raw pointers and the current HIP
stream to the library.  Names follow include/moe_ffn.h.
"""

from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass
from typing import Dict, Optional

import torch

from . import _lib
from ._lib import MoeConfig, MoeGrads, MoeWeights, check, lib


def make_config(T, H, E, I, K, *, act_dtype="bf16", w_dtype="bf16", score_fn="softmax",
                n_group=1, topk_group=1, norm_topk_prob=True, route_scale=1.0,
                swiglu_limit=math.inf, shared_I=0, shared_gated=False, activation="swiglu",
                mx_gemm="decode") -> MoeConfig:
    return MoeConfig(T=T, H=H, E=E, I=I, K=K, act_dtype=_lib.MOE_DTYPE[act_dtype],
                     w_dtype=_lib.MOE_DTYPE[w_dtype], score_fn=_lib.MOE_SCORE[score_fn],
                     n_group=n_group, topk_group=topk_group,
                     norm_topk_prob=int(bool(norm_topk_prob)), route_scale=float(route_scale),
                     swiglu_limit=float(swiglu_limit), shared_I=shared_I,
                     shared_gated=int(bool(shared_gated)), activation=_lib.MOE_ACT[activation],
                     mx_gemm=_lib.MOE_MX_GEMM[mx_gemm])


def config_from_workload(w) -> MoeConfig:
    """MoeConfig of a workloads.Workload."""
    return make_config(w.T, w.H, w.E, w.I, w.K, act_dtype=w.act_dtype, w_dtype=w.w_dtype,
                       score_fn=w.score_fn, n_group=w.n_group, topk_group=w.topk_group,
                       norm_topk_prob=w.norm_topk_prob, route_scale=w.route_scale,
                       swiglu_limit=w.swiglu_limit, shared_I=w.shared_I,
                       shared_gated=w.shared_gated, activation=w.activation, mx_gemm=w.mx_gemm)


def validate(cfg: MoeConfig) -> None:
    check(lib().moe_validate(ctypes.byref(cfg)))


def workspace_bytes(cfg: MoeConfig) -> int:
    n = ctypes.c_size_t(0)
    check(lib().moe_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return int(n.value)


def alloc_workspace(cfg: MoeConfig, device="cuda") -> torch.Tensor:
    """Workspace tensor for `cfg` (torch allocations are 256-byte aligned)."""
    return torch.empty(max(workspace_bytes(cfg), 256), dtype=torch.uint8, device=device)


def _ptr(t: Optional[torch.Tensor], name: str, *, dtype=None, shape=None, device=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _act_dtype(cfg):
    return torch.float32 if cfg.act_dtype == _lib.MOE_DTYPE["f32"] else torch.bfloat16


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


@dataclass
class Routing:
    scores: torch.Tensor    # f32 [T, E]
    indices: torch.Tensor   # int32 [T, K]
    weights: torch.Tensor   # f32 [T, K]
    counts: Optional[torch.Tensor]  # int32 [E]


def route(cfg: MoeConfig, x, gate_w, router_bias=None, expert_bias=None, *, counts=True,
          workspace=None, stream=None, out: Optional[Routing] = None) -> Routing:
    """moe_route: the router's scores, indices, weights (and counts)."""
    dev = x.device
    T, H, E, K = cfg.T, cfg.H, cfg.E, cfg.K
    ad = _act_dtype(cfg)
    if out is None:
        out = Routing(torch.empty(T, E, dtype=torch.float32, device=dev),
                      torch.empty(T, K, dtype=torch.int32, device=dev),
                      torch.empty(T, K, dtype=torch.float32, device=dev),
                      torch.empty(E, dtype=torch.int32, device=dev) if counts else None)
    if workspace is None:
        workspace = alloc_workspace(cfg, dev)
    args = [
        _ptr(x, "x", dtype=ad, shape=(T, H), device=dev),
        _ptr(gate_w, "gate_w", dtype=ad, shape=(E, H), device=dev),
        _ptr(router_bias, "router_bias", dtype=torch.float32, shape=(E,), device=dev),
        _ptr(expert_bias, "expert_bias", dtype=torch.float32, shape=(E,), device=dev),
        _ptr(out.scores, "scores", dtype=torch.float32, shape=(T, E), device=dev),
        _ptr(out.indices, "indices", dtype=torch.int32, shape=(T, K), device=dev),
        _ptr(out.weights, "weights", dtype=torch.float32, shape=(T, K), device=dev),
        _ptr(out.counts, "counts", dtype=torch.int32, shape=(E,), device=dev),
    ]
    check(lib().moe_route(ctypes.byref(cfg), *args, _ptr(workspace, "workspace"),
                          ctypes.c_size_t(workspace.numel()), _stream(stream)))
    return out


class LayerWeights:
    """Device tensors of one layer, in the header's layouts.

    bf16 / f32 experts: w_gate_up [E, 2I, H], w_down [E, H, I].
    MXFP4 experts: w_gate_up uint8 [E, 2I, H/2], w_gate_up_scale uint8
    [E, 2I, H/32], w_down uint8 [E, H, I/2], w_down_scale uint8 [E, H, I/32].
    """

    FIELDS = ("gate_w", "router_bias", "expert_bias", "w_gate_up", "w_down", "w_gate_up_scale",
              "w_down_scale", "b_gate_up", "b_down", "sh_gate_up", "sh_down", "sh_gate")

    def __init__(self, **tensors):
        for f in self.FIELDS:
            setattr(self, f, tensors.pop(f, None))
        if tensors:
            raise TypeError(f"unknown weight fields {sorted(tensors)}")

    def check(self, cfg: MoeConfig, device) -> MoeWeights:
        T, H, E, I, Is = cfg.T, cfg.H, cfg.E, cfg.I, cfg.shared_I
        ad = _act_dtype(cfg)
        mx = cfg.w_dtype == _lib.MOE_DTYPE["mxfp4"]
        wd = {0: torch.float32, 1: torch.bfloat16, 2: torch.uint8}[cfg.w_dtype]
        gu_shape = (E, 2 * I, H // 2) if mx else (E, 2 * I, H)
        dn_shape = (E, H, I // 2) if mx else (E, H, I)
        p = lambda name, **kw: _ptr(getattr(self, name), name, device=device, **kw)
        return MoeWeights(
            gate_w=p("gate_w", dtype=ad, shape=(E, H)),
            router_bias=p("router_bias", dtype=torch.float32, shape=(E,)),
            expert_bias=p("expert_bias", dtype=torch.float32, shape=(E,)),
            w_gate_up=p("w_gate_up", dtype=wd, shape=gu_shape),
            w_down=p("w_down", dtype=wd, shape=dn_shape),
            w_gate_up_scale=p("w_gate_up_scale", dtype=torch.uint8, shape=(E, 2 * I, H // 32)),
            w_down_scale=p("w_down_scale", dtype=torch.uint8, shape=(E, H, I // 32)),
            b_gate_up=p("b_gate_up", dtype=ad, shape=(E, 2 * I)),
            b_down=p("b_down", dtype=ad, shape=(E, H)),
            sh_gate_up=p("sh_gate_up", dtype=ad, shape=(2 * Is, H)),
            sh_down=p("sh_down", dtype=ad, shape=(H, Is)),
            sh_gate=p("sh_gate", dtype=ad, shape=(H,)),
        )


def ffn_forward(cfg: MoeConfig, x: torch.Tensor, weights: LayerWeights, *, out=None,
                routing: Optional[Routing] = None, workspace=None, stream=None):
    """moe_ffn_forward: returns `out` [T, H] (act dtype).  When `routing` is
    given, the router results are also written to its tensors."""
    dev = x.device
    T, H, E, K = cfg.T, cfg.H, cfg.E, cfg.K
    ad = _act_dtype(cfg)
    if out is None:
        out = torch.empty(T, H, dtype=ad, device=dev)
    if workspace is None:
        workspace = alloc_workspace(cfg, dev)
    w = weights.check(cfg, dev)
    r = routing
    rargs = [
        _ptr(r.scores if r else None, "scores", dtype=torch.float32, shape=(T, E), device=dev),
        _ptr(r.indices if r else None, "indices", dtype=torch.int32, shape=(T, K), device=dev),
        _ptr(r.weights if r else None, "weights", dtype=torch.float32, shape=(T, K), device=dev),
        _ptr(r.counts if r else None, "counts", dtype=torch.int32, shape=(E,), device=dev),
    ]
    check(lib().moe_ffn_forward(
        ctypes.byref(cfg), _ptr(x, "x", dtype=ad, shape=(T, H), device=dev), ctypes.byref(w),
        _ptr(out, "out", dtype=ad, shape=(T, H), device=dev), *rargs,
        _ptr(workspace, "workspace"), ctypes.c_size_t(workspace.numel()), _stream(stream)))
    return out


def ffn_forward_noalloc(cfg: MoeConfig, x: torch.Tensor, weights: LayerWeights, *, out: torch.Tensor,
                        routing: Optional[Routing] = None, stream=None):
    """moe_ffn_forward_noalloc: the layer forward on the library's own scratch
    array (no workspace).  `out` (and `routing`, when given) are the caller's;
    this wrapper allocates nothing."""
    dev = x.device
    T, H, E, K = cfg.T, cfg.H, cfg.E, cfg.K
    ad = _act_dtype(cfg)
    w = weights.check(cfg, dev)
    r = routing
    rargs = [
        _ptr(r.scores if r else None, "scores", dtype=torch.float32, shape=(T, E), device=dev),
        _ptr(r.indices if r else None, "indices", dtype=torch.int32, shape=(T, K), device=dev),
        _ptr(r.weights if r else None, "weights", dtype=torch.float32, shape=(T, K), device=dev),
        _ptr(r.counts if r else None, "counts", dtype=torch.int32, shape=(E,), device=dev),
    ]
    check(lib().moe_ffn_forward_noalloc(
        ctypes.byref(cfg), _ptr(x, "x", dtype=ad, shape=(T, H), device=dev), ctypes.byref(w),
        _ptr(out, "out", dtype=ad, shape=(T, H), device=dev), *rargs, _stream(stream)))
    return out


def balance_count(indices: torch.Tensor, tokens_per_expert: torch.Tensor, token_mask=None, *,
                  stream=None) -> torch.Tensor:
    """moe_balance_count: tokens_per_expert [E] int64 += the kept slots of
    `indices` [T, K] int32 (token_mask [T] bool/uint8 keeps tokens; None keeps
    all).  Returns tokens_per_expert."""
    dev = indices.device
    if indices.dim() != 2:
        raise ValueError("indices must be [T, K]")
    T, K = indices.shape
    E = tokens_per_expert.numel()
    if token_mask is not None and token_mask.dtype == torch.bool:
        token_mask = token_mask.view(torch.uint8)
    check(lib().moe_balance_count(
        _ptr(indices, "indices", dtype=torch.int32, device=dev),
        _ptr(token_mask, "token_mask", dtype=torch.uint8, shape=(T,), device=dev),
        T, K, E, _ptr(tokens_per_expert, "tokens_per_expert", dtype=torch.int64, shape=(E,), device=dev),
        _stream(stream)))
    return tokens_per_expert


def balance_update(tokens_per_expert: torch.Tensor, expert_bias: Optional[torch.Tensor],
                   bias_update_rate: float, step_balance: Optional[torch.Tensor] = None, *,
                   stream=None) -> Optional[torch.Tensor]:
    """moe_balance_update: step balance into step_balance [1] f32 (allocated
    when None), the bias sign step on expert_bias [E] f32 in place, and the
    counts zeroed.  Returns step_balance."""
    dev = tokens_per_expert.device
    E = tokens_per_expert.numel()
    if step_balance is None:
        step_balance = torch.empty(1, dtype=torch.float32, device=dev)
    check(lib().moe_balance_update(
        _ptr(tokens_per_expert, "tokens_per_expert", dtype=torch.int64, shape=(E,), device=dev),
        _ptr(expert_bias, "expert_bias", dtype=torch.float32, shape=(E,), device=dev),
        E, ctypes.c_float(bias_update_rate),
        _ptr(step_balance, "step_balance", dtype=torch.float32, shape=(1,), device=dev),
        _stream(stream)))
    return step_balance


@dataclass
class Grads:
    """f32 gradients of sum(out * dout) (moe_ffn_backward); None where the
    layer has no such input."""
    dx: torch.Tensor
    dgate: torch.Tensor
    dw_gate_up: torch.Tensor
    dw_down: torch.Tensor
    drouter_bias: Optional[torch.Tensor] = None
    db_gate_up: Optional[torch.Tensor] = None
    db_down: Optional[torch.Tensor] = None
    dsh_gate_up: Optional[torch.Tensor] = None
    dsh_down: Optional[torch.Tensor] = None
    dsh_gate: Optional[torch.Tensor] = None


def backward_workspace_bytes(cfg: MoeConfig) -> int:
    n = ctypes.c_size_t()
    check(lib().moe_backward_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def ffn_backward(cfg: MoeConfig, x: torch.Tensor, weights: LayerWeights, dout: torch.Tensor,
                 routing: Routing, *, workspace=None, stream=None) -> Grads:
    """moe_ffn_backward: gradients of sum(out * dout) at the forward whose
    scores and indices are in `routing`."""
    dev = x.device
    T, H, E, I, K, Is = cfg.T, cfg.H, cfg.E, cfg.I, cfg.K, cfg.shared_I
    ad = _act_dtype(cfg)
    w = weights.check(cfg, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    g = Grads(torch.empty(T, H, **f32), torch.empty(E, H, **f32), torch.empty(E, 2 * I, H, **f32),
              torch.empty(E, H, I, **f32))
    if weights.router_bias is not None:
        g.drouter_bias = torch.empty(E, **f32)
    if weights.b_gate_up is not None:
        g.db_gate_up = torch.empty(E, 2 * I, **f32)
    if weights.b_down is not None:
        g.db_down = torch.empty(E, H, **f32)
    if Is > 0:
        g.dsh_gate_up = torch.empty(2 * Is, H, **f32)
        g.dsh_down = torch.empty(H, Is, **f32)
        if cfg.shared_gated:
            g.dsh_gate = torch.empty(H, **f32)
    if workspace is None:
        workspace = torch.empty(max(backward_workspace_bytes(cfg), 256), dtype=torch.uint8, device=dev)
    cg = MoeGrads(**{f: (_ptr(getattr(g, f), f).value if getattr(g, f) is not None else None)
                     for f, _ in MoeGrads._fields_})
    check(lib().moe_ffn_backward(
        ctypes.byref(cfg), _ptr(x, "x", dtype=ad, shape=(T, H), device=dev), ctypes.byref(w),
        _ptr(dout, "dout", dtype=ad, shape=(T, H), device=dev),
        _ptr(routing.scores, "scores", dtype=torch.float32, shape=(T, E), device=dev),
        _ptr(routing.indices, "indices", dtype=torch.int32, shape=(T, K), device=dev),
        ctypes.byref(cg), _ptr(workspace, "workspace"), ctypes.c_size_t(workspace.numel()), _stream(stream)))
    return g


def empty_routing(cfg: MoeConfig, device="cuda") -> Routing:
    return Routing(torch.empty(cfg.T, cfg.E, dtype=torch.float32, device=device),
                   torch.empty(cfg.T, cfg.K, dtype=torch.int32, device=device),
                   torch.empty(cfg.T, cfg.K, dtype=torch.float32, device=device),
                   torch.empty(cfg.E, dtype=torch.int32, device=device))


def layer_weights_from_workload(w, device="cuda") -> LayerWeights:
    """Draw a workload's weights directly on `device` (seeded, synthetic)."""
    from . import workloads as W
    experts = W.gen_experts_stacked(w, device)
    shared = W.gen_shared(w, device) or {}
    if w.w_dtype == "mxfp4":
        ex = dict(w_gate_up=experts["codes_gate_up"], w_gate_up_scale=experts["scales_gate_up"],
                  w_down=experts["codes_down"], w_down_scale=experts["scales_down"])
    else:
        ex = dict(w_gate_up=experts["w_gate_up"], w_down=experts["w_down"])
    if "b_gate_up" in experts:
        ex["b_gate_up"] = experts["b_gate_up"]
        ex["b_down"] = experts["b_down"]
    return LayerWeights(gate_w=W.gen_gate(w, device), router_bias=W.gen_router_bias(w, device),
                        expert_bias=W.gen_expert_bias(w, device), **ex, **shared)
