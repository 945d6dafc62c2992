"""Seeded synthetic workloads for the MoE FFN layer: shapes and input draws.

This module holds no arithmetic of the layer itself.  It describes the five
workload families (shapes, dtypes, routing options, value distributions) and
draws their inputs from a counter-based generator that gives bit-identical
values on the CPU and on the GPU, so that any slice (one expert, one token)
can be regenerated on the host for checking without copying it back from the
device.

Generator
  u32(seed, tensor_id, slice_id, i) = fmix32(fmix32(i + key) ^ key2), where
  fmix32 is the MurmurHash3 32-bit finaliser and key/key2 are fmix32-mixed
  combinations of (seed, tensor_id, slice_id).  All integer arithmetic is
  modulo 2**32 and runs in int64 torch ops with explicit masking.
  Normal draws: the upper 16 bits index a fixed table of the 65536 standard
  normal quantiles ndtri((j + 0.5) / 65536) (computed once on the CPU in fp64,
  rounded to fp32), times std in fp32, then rounded to bf16 by integer
  round-to-nearest-even where the tensor is bf16.  The draw is a 65536-point
  discretised N(0, std^2), truncated at about 4.3 std.
  Byte draws (MXFP4 codes) take bits 8..15; E8M0 scale draws are
  127 + lo + (u32 mod (hi - lo + 1)).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import numpy as np
import torch

MASK32 = 0xFFFFFFFF

# tensor ids of the generator (fixed; part of the workload definition)
TID = {
    "x": 1, "gate": 2, "router_bias": 3, "expert_bias": 4,
    "w_gate_up": 5, "w_down": 6, "b_gate_up": 7, "b_down": 8,
    "sh_gate_up": 9, "sh_down": 10, "sh_gate": 11,
    "codes_gate_up": 12, "codes_down": 13, "scales_gate_up": 14, "scales_down": 15,
    "balance_indices": 16, "token_mask": 17, "balance_bias": 18, "dout": 19,
}


def _mulmod32(h: torch.Tensor, c: int) -> torch.Tensor:
    """(h * c) mod 2**32 for 0 <= h, c < 2**32 without int64 overflow."""
    lo, hi = c & 0xFFFF, c >> 16
    return (h * lo + (((h * hi) & 0xFFFF) << 16)) & MASK32


def _fmix32(h: torch.Tensor) -> torch.Tensor:
    h = h & MASK32
    h = h ^ (h >> 16)
    h = _mulmod32(h, 0x85EBCA6B)
    h = h ^ (h >> 13)
    h = _mulmod32(h, 0xC2B2AE35)
    h = h ^ (h >> 16)
    return h


def _fmix32_int(h: int) -> int:
    h &= MASK32
    h ^= h >> 16
    h = (h * 0x85EBCA6B) & MASK32
    h ^= h >> 13
    h = (h * 0xC2B2AE35) & MASK32
    h ^= h >> 16
    return h


def _keys(seed: int, tid: int, sid: int):
    k1 = _fmix32_int((seed * 0x9E3779B1 + tid * 0x85EBCA77 + sid * 0xC2B2AE3D + 0x27D4EB2F) & MASK32)
    k2 = _fmix32_int((k1 ^ (tid * 0x165667B1) ^ (sid * 0x27D4EB2F) ^ 0x61C88647) & MASK32)
    return k1, k2


def _fmix32_np(h: np.ndarray) -> np.ndarray:
    """fmix32 on uint32 arrays (numpy wraps uint32 products modulo 2**32)."""
    h = h ^ (h >> np.uint32(16))
    h = h * np.uint32(0x85EBCA6B)
    h = h ^ (h >> np.uint32(13))
    h = h * np.uint32(0xC2B2AE35)
    h = h ^ (h >> np.uint32(16))
    return h


def _u32_np(seed: int, tid: int, sid: int, n: int) -> np.ndarray:
    k1, k2 = _keys(seed, tid, sid)
    with np.errstate(over="ignore"):
        i = np.arange(n, dtype=np.uint32)
        return _fmix32_np(_fmix32_np(i + np.uint32(k1)) ^ np.uint32(k2))


def draw_u32(seed: int, tid: int, sid: int, n: int, device="cpu") -> torch.Tensor:
    """n counter-based 32-bit draws (int64 tensor holding values < 2**32).

    The CPU path runs the arithmetic in numpy uint32, the device path in torch
    int64 with masking; both compute the same integers."""
    if torch.device(device).type == "cpu":
        return torch.from_numpy(_u32_np(seed, tid, sid, n).astype(np.int64))
    k1, k2 = _keys(seed, tid, sid)
    i = torch.arange(n, dtype=torch.int64, device=device)
    return _fmix32(_fmix32(i + k1) ^ k2)


_TABLE: Dict[str, torch.Tensor] = {}


def normal_table(device="cpu") -> torch.Tensor:
    """fp32 [65536]: standard normal quantiles at the bin centres."""
    key = str(device)
    if key not in _TABLE:
        if "cpu" not in _TABLE:
            p = (torch.arange(65536, dtype=torch.float64) + 0.5) / 65536.0
            _TABLE["cpu"] = torch.special.ndtri(p).to(torch.float32)
        _TABLE[key] = _TABLE["cpu"].to(device)
    return _TABLE[key]


def draw_normal_f32(seed, tid, sid, n, std, device="cpu") -> torch.Tensor:
    if torch.device(device).type == "cpu":
        z = normal_table("cpu").numpy()[_u32_np(seed, tid, sid, n) >> np.uint32(16)]
        return torch.from_numpy(z * np.float32(std))
    u = draw_u32(seed, tid, sid, n, device)
    z = normal_table(device)[(u >> 16)]
    return z * torch.tensor(std, dtype=torch.float32, device=device)


def f32_to_bf16_bits(v: torch.Tensor) -> torch.Tensor:
    """Round fp32 -> bf16 (nearest, ties to even) by integer ops; returns the
    16-bit patterns as an int64 tensor.  Inputs are finite."""
    if v.device.type == "cpu":
        b = np.ascontiguousarray(v.numpy()).view(np.uint32)
        with np.errstate(over="ignore"):
            r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        return torch.from_numpy(r.astype(np.int64))
    b = v.contiguous().view(torch.int32).to(torch.int64) & MASK32
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return r & 0xFFFF


def bits_to_bf16_tensor(bits: torch.Tensor) -> torch.Tensor:
    """int64 bf16 patterns -> torch.bfloat16 tensor on the same device."""
    if bits.device.type == "cpu":
        return torch.from_numpy(bits.numpy().astype(np.uint16).view(np.int16)).view(torch.bfloat16)
    signed = torch.where(bits >= 32768, bits - 65536, bits)
    return signed.to(torch.int16).view(torch.bfloat16)


def draw_bf16(seed, tid, sid, n, std, device="cpu") -> torch.Tensor:
    return bits_to_bf16_tensor(f32_to_bf16_bits(draw_normal_f32(seed, tid, sid, n, std, device)))


def draw_bytes(seed, tid, sid, n, device="cpu") -> torch.Tensor:
    return ((draw_u32(seed, tid, sid, n, device) >> 8) & 0xFF).to(torch.uint8)


def draw_e8m0(seed, tid, sid, n, lo, hi, device="cpu") -> torch.Tensor:
    u = draw_u32(seed, tid, sid, n, device)
    return (127 + lo + (u % (hi - lo + 1))).to(torch.uint8)


# ----------------------------------------------------------------------------
# Workload descriptions
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    """One MoE FFN layer configuration and its input distribution."""
    name: str
    T: int
    H: int
    E: int
    I: int
    K: int
    act_dtype: str = "bf16"            # x, router gate, shared expert, out: "f32" | "bf16"
    w_dtype: str = "bf16"              # routed experts: "f32" | "bf16" | "mxfp4"
    score_fn: str = "softmax"
    n_group: int = 1
    topk_group: int = 1
    norm_topk_prob: bool = True
    route_scale: float = 1.0
    swiglu_limit: float = math.inf
    activation: str = "swiglu"         # "swiglu" | "swiglu_oai" (gpt-oss's swigluoai)
    mx_gemm: str = "decode"            # MXFP4 gate_up at large T: "decode" | "block_scaled"
    shared_I: int = 0
    shared_gated: bool = False
    x_std: float = 1.0
    w_std: float = 0.02
    expert_bias_std: float = 0.0       # selection-only bias; 0 = absent
    router_bias_std: float = 0.0       # logit bias; 0 = absent
    expert_linear_bias_std: float = 0.0  # gpt-oss-style per-expert linear biases; 0 = absent
    mx_scale_lo: int = -3              # E8M0 scales are 127 + U{lo..hi}
    mx_scale_hi: int = 0
    seed: int = 0

    def with_T(self, T: int) -> "Workload":
        return replace(self, T=T)

    @property
    def torch_act_dtype(self):
        return torch.float32 if self.act_dtype == "f32" else torch.bfloat16


def _c1():
    return Workload("tiny_f32_e8_top2", T=64, H=256, E=8, I=128, K=2,
                    act_dtype="f32", w_dtype="f32")


def _c2(T=72):
    return Workload("qwen3_8b_moe_draft_e8_top1", T=T, H=4096, E=8, I=1536, K=1)


def _c3(T=72, selection_bias=False):
    # The drafter's "router bias ~ N(0, 0.1)" in its two readings: a logit
    # bias added to the fp32 router logits (moves selection and weights), or
    # the selection-only expert bias (moves the picks only).  At std 0.1 the
    # selection-only bias dominates softmax scores of about 1/E = 0.002, so
    # that reading routes most tokens to the same few experts (collapsed
    # routing: a few dozen active experts, the largest holding every token).
    if selection_bias:
        return Workload("qwen3_5_moe_drafter_e512_top10_selbias", T=T, H=5120, E=512,
                        I=512, K=10, shared_I=2048, shared_gated=True, expert_bias_std=0.1)
    return Workload("qwen3_5_moe_drafter_e512_top10", T=T, H=5120, E=512, I=512, K=10,
                    shared_I=2048, shared_gated=True, router_bias_std=0.1)


def _c4(T=72, score_fn="sigmoid"):
    return Workload(f"deepseek_v4_style_e256_top8_{score_fn}", T=T, H=4096, E=256, I=2048,
                    K=8, score_fn=score_fn, n_group=8, topk_group=4, route_scale=2.5,
                    swiglu_limit=7.0, shared_I=2048, shared_gated=False,
                    expert_bias_std=0.05)


def _c5(T=72, activation="swiglu", mx_gemm="decode"):
    # activation "swiglu_oai": the same experts with gpt-oss's own activation;
    # mx_gemm "block_scaled": the large-T gate_up on the block-scaled matrix cores
    name = ("gpt_oss_style_mxfp4_e32_top4" + ("_oai" if activation == "swiglu_oai" else "")
            + ("_blockscaled" if mx_gemm == "block_scaled" else ""))
    return Workload(name, T=T, H=2880, E=32, I=2880, K=4, w_dtype="mxfp4", swiglu_limit=7.0,
                    activation=activation, expert_linear_bias_std=0.02, mx_gemm=mx_gemm)


WORKLOADS = {
    "tiny_f32": _c1,
    "qwen3_8b_moe_draft": _c2,
    "qwen3_5_moe_drafter": _c3,
    "deepseek_v4_style": _c4,
    "gpt_oss_style_mxfp4": _c5,
}

# (family, T) pairs at the sizes the workloads are quoted on
FULL_CASES = [
    ("tiny_f32", {}),
    ("qwen3_8b_moe_draft", {"T": 72}), ("qwen3_8b_moe_draft", {"T": 8192}),
    ("qwen3_5_moe_drafter", {"T": 72}), ("qwen3_5_moe_drafter", {"T": 4096}),
    ("qwen3_5_moe_drafter", {"T": 72, "selection_bias": True}),
    ("qwen3_5_moe_drafter", {"T": 4096, "selection_bias": True}),
    ("deepseek_v4_style", {"T": 72, "score_fn": "sigmoid"}),
    ("deepseek_v4_style", {"T": 4096, "score_fn": "sigmoid"}),
    ("deepseek_v4_style", {"T": 72, "score_fn": "sqrtsoftplus"}),
    ("deepseek_v4_style", {"T": 4096, "score_fn": "sqrtsoftplus"}),
    ("gpt_oss_style_mxfp4", {"T": 72}), ("gpt_oss_style_mxfp4", {"T": 2048}),
    ("gpt_oss_style_mxfp4", {"T": 72, "activation": "swiglu_oai"}),
    ("gpt_oss_style_mxfp4", {"T": 2048, "activation": "swiglu_oai"}),
    ("gpt_oss_style_mxfp4", {"T": 2048, "mx_gemm": "block_scaled"}),
]


def workload(family: str, **kw) -> Workload:
    return WORKLOADS[family](**kw)


# ----------------------------------------------------------------------------
# Tensors
# ----------------------------------------------------------------------------

def _act(w: Workload, tid: str, sid: int, n: int, std: float, device):
    if w.act_dtype == "f32":
        return draw_normal_f32(w.seed, TID[tid], sid, n, std, device)
    return draw_bf16(w.seed, TID[tid], sid, n, std, device)


def gen_x(w: Workload, device="cpu") -> torch.Tensor:
    """x [T, H]; slice id = T so that each token count has its own draw."""
    return _act(w, "x", w.T, w.T * w.H, w.x_std, device).view(w.T, w.H)


def gen_gate(w: Workload, device="cpu") -> torch.Tensor:
    return _act(w, "gate", 0, w.E * w.H, w.w_std, device).view(w.E, w.H)


def gen_expert_bias(w: Workload, device="cpu") -> Optional[torch.Tensor]:
    if w.expert_bias_std == 0:
        return None
    return draw_normal_f32(w.seed, TID["expert_bias"], 0, w.E, w.expert_bias_std, device)


def gen_router_bias(w: Workload, device="cpu") -> Optional[torch.Tensor]:
    if w.router_bias_std == 0:
        return None
    return draw_normal_f32(w.seed, TID["router_bias"], 0, w.E, w.router_bias_std, device)


def gen_expert(w: Workload, e: int, device="cpu") -> dict:
    """Expert e's routed weights in storage format.

    bf16/f32: {"w_gate_up": [2I, H], "w_down": [H, I]}.
    mxfp4:    {"codes_gate_up": u8 [2I, H/2], "scales_gate_up": u8 [2I, H/32],
               "codes_down": u8 [H, I/2], "scales_down": u8 [H, I/32]}.
    plus {"b_gate_up": [2I], "b_down": [H]} (act dtype) when the workload has
    per-expert linear biases.
    """
    H, I = w.H, w.I
    out = {}
    if w.w_dtype in ("bf16", "f32"):
        mk = draw_bf16 if w.w_dtype == "bf16" else draw_normal_f32
        out["w_gate_up"] = mk(w.seed, TID["w_gate_up"], e, 2 * I * H, w.w_std, device).view(2 * I, H)
        out["w_down"] = mk(w.seed, TID["w_down"], e, H * I, w.w_std, device).view(H, I)
    elif w.w_dtype == "mxfp4":
        out["codes_gate_up"] = draw_bytes(w.seed, TID["codes_gate_up"], e, 2 * I * H // 2, device).view(2 * I, H // 2)
        out["scales_gate_up"] = draw_e8m0(w.seed, TID["scales_gate_up"], e, 2 * I * H // 32,
                                          w.mx_scale_lo, w.mx_scale_hi, device).view(2 * I, H // 32)
        out["codes_down"] = draw_bytes(w.seed, TID["codes_down"], e, H * I // 2, device).view(H, I // 2)
        out["scales_down"] = draw_e8m0(w.seed, TID["scales_down"], e, H * I // 32,
                                       w.mx_scale_lo, w.mx_scale_hi, device).view(H, I // 32)
    else:
        raise ValueError(w.w_dtype)
    if w.expert_linear_bias_std:
        out["b_gate_up"] = _act(w, "b_gate_up", e, 2 * I, w.expert_linear_bias_std, device)
        out["b_down"] = _act(w, "b_down", e, H, w.expert_linear_bias_std, device)
    return out


def gen_shared(w: Workload, device="cpu") -> Optional[dict]:
    if not w.shared_I:
        return None
    Is, H = w.shared_I, w.H
    out = {
        "sh_gate_up": _act(w, "sh_gate_up", 0, 2 * Is * H, w.w_std, device).view(2 * Is, H),
        "sh_down": _act(w, "sh_down", 0, H * Is, w.w_std, device).view(H, Is),
    }
    if w.shared_gated:
        out["sh_gate"] = _act(w, "sh_gate", 0, H, w.w_std, device)
    return out


def gen_experts_stacked(w: Workload, device="cpu") -> dict:
    """All experts stacked along a leading E axis, built one expert at a time
    directly on `device` (no host copy of the whole stack)."""
    first = gen_expert(w, 0, device)
    stacked = {k: torch.empty((w.E,) + tuple(v.shape), dtype=v.dtype, device=device)
               for k, v in first.items()}
    for k, v in first.items():
        stacked[k][0].copy_(v)
    del first
    for e in range(1, w.E):
        for k, v in gen_expert(w, e, device).items():
            stacked[k][e].copy_(v)
    return stacked


def to_numpy_storage(t: torch.Tensor) -> np.ndarray:
    """Storage-format tensor -> numpy: bf16 as uint16 bit patterns, f32 as
    float32, u8 as uint8."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def algorithmic_bytes(w: Workload, counts: np.ndarray) -> dict:
    """Bytes a forward must move at least once, given the expert counts.

    Weights of active experts (+ MXFP4 scales, + linear biases), the router
    gate, the shared expert, the activations in and out, and the router
    outputs (scores, indices, weights).  Intermediates are excluded.
    """
    act = 4 if w.act_dtype == "f32" else 2
    active = int((np.asarray(counts) > 0).sum())
    H, I, E, T, K = w.H, w.I, w.E, w.T, w.K
    if w.w_dtype == "mxfp4":
        gu = 2 * I * H // 2 + 2 * I * H // 32
        dn = H * I // 2 + H * I // 32
    else:
        wb = 4 if w.w_dtype == "f32" else 2
        gu = 2 * I * H * wb
        dn = H * I * wb
    lin_b = (2 * I + H) * act if w.expert_linear_bias_std else 0
    expert = active * (gu + dn + lin_b)
    router = E * H * act
    shared = (3 * w.shared_I * H * act + (H * act if w.shared_gated else 0)) if w.shared_I else 0
    io = 2 * T * H * act + T * E * 4 + T * K * 8
    return {"gate_up": active * (gu + (2 * I * act if lin_b else 0)),
            "down": active * (dn + (H * act if lin_b else 0)),
            "expert": expert, "router": router, "shared": shared, "io": io,
            "total": expert + router + shared + io}


def algorithmic_flops(w: Workload) -> dict:
    """2 flops per multiply-add of the layer's contractions."""
    T, H, I, E, K = w.T, w.H, w.I, w.E, w.K
    routed = 6 * T * K * H * I
    shared = 6 * T * H * w.shared_I
    router = 2 * T * E * H + (2 * T * H if w.shared_gated else 0)
    return {"gate_up": 4 * T * K * H * I, "down": 2 * T * K * H * I,
            "routed": routed, "shared": shared, "router": router,
            "total": routed + shared + router}


def gen_balance_inputs(seed: int, T: int, K: int, E: int, skew: float = 1.0, keep: float = 1.0,
                       sid: int = 0):
    """Synthetic routing for the load-balancing state: expert ids [T, K] int32
    (id = floor(E * u^skew) for uniform u, so skew > 1 crowds the low ids, as a
    collapsing router would), a kept-token mask [T] bool (keep = fraction
    kept; 1 keeps all) and an fp32 bias [E] ~ N(0, 0.01).  CPU tensors."""
    u = draw_u32(seed, TID["balance_indices"], sid, T * K).double() / 4294967296.0
    idx = torch.clamp((E * u.pow(skew)).floor(), max=E - 1).to(torch.int32).view(T, K)
    m = draw_u32(seed, TID["token_mask"], sid, T).double() / 4294967296.0
    mask = m < keep
    bias = draw_normal_f32(seed, TID["balance_bias"], sid, E, 0.01)
    return idx, mask, bias


def gen_dout(w: Workload, device="cpu") -> torch.Tensor:
    """Output gradient [T, H] for the backward, ~ N(0, 1) in the activation dtype."""
    return _act(w, "dout", 0, w.T * w.H, 1.0, device).view(w.T, w.H)

