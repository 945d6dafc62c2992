"""Plain CPU oracle for the MoE FFN layer forward of DFlash/DSpark draft models.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check of the repository's entry
module and the CPU-baseline leg of the benchmark do.  It shares no code with
the HIP library and does not import the product package; it takes plain numpy
arrays (bf16 tensors as their uint16 bit patterns) and returns numpy arrays.

Every step is the plain definition, written so that it can be checked against
the pages by eye.  Floating point is fp64 except where the pages fix fp32
(router logits, scores, the selection values and the combine weights are fp32
per the router contract), in which case the value is computed in fp64 and
rounded once to fp32, or, for the short fp32 chains the pages spell out
(choice = score + bias, the renormalisation), computed in fp32 directly.

Pages cited (title and section; no other source):
  [SF1033]  SpecForge PR #1033 "MoE FFN for DFlash-family drafts: the module"
            -- "Router" section (table with rows score / select /
            routing_weights), and its commit notes.
  [SF1073]  SpecForge PR #1073 "MoE drafts: DeepSeek-V4.1's own DSpark draft
            (stacked on #1035)" -- commit notes: the fp32 expert_bias, select on
            shifted scores, the DeepSeek-V4 family, the V4.1 converter.
  [SGL48763] sglang PR #48763 "[Feat] dflash: Serve MoE FFN drafts for DFlash
            and DSpark" -- Modifications, Verification, commit notes on the
            DraftMLP / DraftMoE forward and on the CUDA fixes.
  [SF941]   SpecForge PR #941 "feat(serving): SGLang draft classes for the
            Qwen3.8-27B DSpark MoE drafter (SGLang FusedMoE path) + tuned
            fused-MoE configs" -- "What" and "Validation" sections, follow-up
            comment on DeepSeek-V4 drafters.
  [MI143]   MoE-Infinity PR #143 "feat(dflash): converge DFlash spec-decode
            stack -> dev (supersedes #140)" -- commit note on loading the
            resident gpt-oss MXFP4 experts.

Readings taken where the pages leave a step open are marked READING; each is
listed in the design notes of the repository.  Pins: every function below is
pinned by a test in tests/test_oracle_pins.py against brute force, closed
forms, library routines or the invariants the pages state.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Callable, Optional

import numpy as np

F32 = np.float32
F64 = np.float64

# [SF1033] commit note on the renormalisation epsilon: the top-k sum is guarded
# with 1e-20 (the DeepSeek / torchtitan value), added in fp32.
RENORM_EPS = F32(1e-20)

SCORE_FNS = ("softmax", "sigmoid", "sqrtsoftplus")


# ----------------------------------------------------------------------------
# Number formats
# ----------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values.

    A bf16 value is the upper half of an IEEE binary32 word, so widening the
    bits by 16 zero bits gives the fp32 value, which fp64 holds exactly.
    """
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(F64)


def e2m1_to_f64(code: np.ndarray) -> np.ndarray:
    """OCP Microscaling FP4 (E2M1) element code 0..15 -> float64.

    Bit 3 is the sign, bits 2..1 the exponent (bias 1), bit 0 the mantissa.
    Exponent 0 is subnormal: 0.5 * m.  Otherwise 2**(e-1) * (1 + m/2).
    """
    code = np.asarray(code, dtype=np.int64)
    sign = np.where((code >> 3) & 1, -1.0, 1.0)
    e = (code >> 1) & 3
    m = code & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, (e - 1).astype(np.int32)))
    return sign * mag


def e8m0_to_f64(scale: np.ndarray) -> np.ndarray:
    """OCP Microscaling E8M0 shared scale 0..254 -> 2**(s-127) (255 is NaN)."""
    s = np.asarray(scale, dtype=np.int64)
    out = np.ldexp(np.ones(s.shape, dtype=F64), (s - 127).astype(np.int32))
    return np.where(s == 255, np.nan, out)


def mxfp4_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Packed MXFP4 weight matrix -> float64 [N, Kin].

    Layout per [MI143] (commit note on the resident gpt-oss experts): blocks
    are output-major, codes [N, Kin/2] uint8 and scales [N, Kin/32] uint8,
    used without a transpose.  Packing per [SF1073] (V4.1 converter commit
    note): two E2M1 codes per byte along the input dimension, low nibble
    first, one E8M0 scale per 32 inputs.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    n, half = codes.shape
    kin = 2 * half
    assert scales.shape == (n, kin // 32), (scales.shape, n, kin)
    elem = np.empty((n, kin), dtype=np.uint8)
    elem[:, 0::2] = codes & 0x0F      # even input index: low nibble
    elem[:, 1::2] = codes >> 4        # odd input index: high nibble
    vals = e2m1_to_f64(elem)
    scale_per_elem = np.repeat(e8m0_to_f64(scales), 32, axis=1)
    return vals * scale_per_elem


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Activation / weight tensor in its storage format -> float64."""
    if dtype == "bf16":
        return bf16_to_f64(a)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(F64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# Router: score -> select -> routing_weights   ([SF1033] "Router" table)
# ----------------------------------------------------------------------------

def router_logits(x64: np.ndarray, gate64: np.ndarray,
                  router_bias: Optional[np.ndarray] = None) -> np.ndarray:
    """fp32 router logits [T, E] = x [T,H] . gate [E,H]^T.

    [SF1033] "Router" table, row score: a linear gate weight [E, H].
    [SGL48763] DraftMoE forward commit note and [SF941] "What": the logits
    reach top-k in fp32.  READING: the products of bf16 (or fp32) inputs are
    exact in fp64; the fp64 sum is rounded once to fp32.  The optional
    router_bias (the logit-bias variant of the qwen3_5_moe recipe, [SF941]
    "What") is one fp32 add after that rounding.
    """
    logits = (x64 @ gate64.T).astype(F32)
    if router_bias is not None:
        logits = (logits + np.asarray(router_bias, dtype=F32)).astype(F32)
    return logits


def score(logits32: np.ndarray, fn: str) -> np.ndarray:
    """fp32 scores [T, E] from fp32 logits, evaluated in fp64, rounded once.

    softmax: [SF1033] "Router" table, row score (probabilities in [0, 1]).
    sigmoid: [SF1033] text under the table (DeepSeek-V4 as TopKRouter with
             score_fn sigmoid).
    sqrtsoftplus: [SF1073] DeepSeek-V4 family commit note (sqrt of softplus
             scores); softplus written in its overflow-free form
             max(l, 0) + log1p(exp(-|l|)).
    """
    l = np.asarray(logits32, dtype=F32).astype(F64)
    if fn == "softmax":
        z = np.exp(l - l.max(axis=-1, keepdims=True))
        s = z / z.sum(axis=-1, keepdims=True)
    elif fn == "sigmoid":
        s = 1.0 / (1.0 + np.exp(-l))
    elif fn == "sqrtsoftplus":
        s = np.sqrt(np.maximum(l, 0.0) + np.log1p(np.exp(-np.abs(l))))
    else:
        raise ValueError(fn)
    return s.astype(F32)


def choice(scores32: np.ndarray, expert_bias: Optional[np.ndarray]) -> np.ndarray:
    """Selection values: scores shifted by the fp32 expert_bias (one fp32 add).

    [SF1073] expert-bias commit note: an fp32 expert_bias moves the top-k picks
    and never the weights; select-on-shifted-scores commit note: select gets
    the shifted scores.
    """
    s = np.asarray(scores32, dtype=F32)
    if expert_bias is None:
        return s.copy()
    return (s + np.asarray(expert_bias, dtype=F32)).astype(F32)


def topk_desc(values32: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest values, largest first; equal values go to the
    lower index (READING: the pages state no tie rule; lowest index wins).

    A stable ascending sort of the negated values keeps equal values in index
    order, which is exactly that rule (negation of an fp32 value is exact).
    """
    v = np.asarray(values32, dtype=F32)
    order = np.argsort(-v, kind="stable")
    return order[:k].astype(np.int32)


def group_scores(choice_row32: np.ndarray, n_group: int) -> np.ndarray:
    """Per-group score for group-limited selection: sum of the two largest
    selection values inside the group, one fp32 add.

    [SF1033] "Router" table, row select (DeepSeek-V3's group-limited top-k as a
    select override).  READING: the DeepSeek-V3 group score (top-2 sum) over
    the bias-shifted values, per [SF1073] (select sees only shifted scores).
    """
    c = np.asarray(choice_row32, dtype=F32)
    e = c.shape[-1]
    g = c.reshape(n_group, e // n_group)
    two = -np.sort(-g, axis=-1)[:, :2]          # two largest per group
    return (two[:, 0] + two[:, 1]).astype(F32)


def select(choice32: np.ndarray, k: int, n_group: int = 1, topk_group: int = 1) -> np.ndarray:
    """indices [T, K] int32 from selection values [T, E].

    Plain: top-k of the selection values.  Group-limited (n_group > 1): keep
    the topk_group groups with the largest group score (ties to the lower
    group), drop every expert of the other groups, then plain top-k over what
    is left.  [SF1033] "Router" table, row select.
    """
    c = np.asarray(choice32, dtype=F32)
    t_count, e = c.shape
    out = np.empty((t_count, k), dtype=np.int32)
    for t in range(t_count):
        row = c[t]
        if n_group > 1:
            gs = group_scores(row, n_group)
            keep = topk_desc(gs, topk_group)
            size = e // n_group
            masked = np.full(e, -np.inf, dtype=F32)
            for g in keep:
                masked[g * size:(g + 1) * size] = row[g * size:(g + 1) * size]
            row = masked
        out[t] = topk_desc(row, k)
    return out


def routing_weights(scores32: np.ndarray, indices: np.ndarray, norm_topk_prob: bool,
                    route_scale: float, eps=RENORM_EPS) -> np.ndarray:
    """weights [T, K] fp32.

    [SF1033] "Router" table, row routing_weights: gather from the UNSHIFTED
    scores; renormalise by their sum when norm_topk_prob, with the 1e-20 guard
    (commit note on the epsilon); then multiply by route_scale.  READING: the
    sum runs in fp32 in output order (k = 0..K-1), the guard is added to the
    sum, the division comes before the scale.
    """
    s = np.asarray(scores32, dtype=F32)
    idx = np.asarray(indices)
    t_count, k = idx.shape
    rs = F32(route_scale)
    w = np.empty((t_count, k), dtype=F32)
    for t in range(t_count):
        picked = s[t, idx[t]]
        if norm_topk_prob:
            total = F32(0.0)
            for v in picked:
                total = F32(total + v)
            denom = F32(total + F32(eps))
            w[t] = (picked / denom).astype(F32) * rs
        else:
            w[t] = picked * rs
    return w.astype(F32)


@dataclass
class RouteResult:
    logits: np.ndarray    # fp32 [T, E] (after the optional logit bias)
    scores: np.ndarray    # fp32 [T, E], unshifted
    choice: np.ndarray    # fp32 [T, E], scores + expert_bias
    indices: np.ndarray   # int32 [T, K]
    weights: np.ndarray   # fp32 [T, K]


def route(x64, gate64, *, k, score_fn="softmax", n_group=1, topk_group=1,
          norm_topk_prob=True, route_scale=1.0, expert_bias=None,
          router_bias=None) -> RouteResult:
    """The Router's fixed forward: score -> select -> routing_weights.

    [SF1033] "Router" section: forward is fixed and returns scores, indices,
    weights; the bias is applied between score and select ([SF1073]).
    """
    lg = router_logits(x64, gate64, router_bias)
    sc = score(lg, score_fn)
    ch = choice(sc, expert_bias)
    idx = select(ch, k, n_group, topk_group)
    w = routing_weights(sc, idx, norm_topk_prob, route_scale)
    return RouteResult(lg, sc, ch, idx, w)


def selection_margins(choice32: np.ndarray, indices: np.ndarray, n_group: int = 1,
                      topk_group: int = 1) -> np.ndarray:
    """Per-token distance of the selection from its nearest tie [T] (fp64).

    The gap between the K-th picked value and the best value not picked among
    the admissible experts and, for group-limited selection, the gap between
    the last kept group score and the best dropped one.  A token whose margin
    is larger than the fp32 rounding differences of two implementations has
    one correct top-k; a smaller margin marks a near-tie.
    """
    c = np.asarray(choice32, dtype=F32).astype(F64)
    t_count, e = c.shape
    k = indices.shape[1]
    out = np.empty(t_count, dtype=F64)
    for t in range(t_count):
        row = c[t].copy()
        m = np.inf
        if n_group > 1:
            gs = group_scores(c[t].astype(F32), n_group).astype(F64)
            order = np.argsort(-gs, kind="stable")
            if topk_group < n_group:
                m = min(m, gs[order[topk_group - 1]] - gs[order[topk_group]])
            size = e // n_group
            allowed = np.zeros(e, dtype=bool)
            for g in order[:topk_group]:
                allowed[g * size:(g + 1) * size] = True
            row[~allowed] = -np.inf
        picked = row[indices[t]]
        rest = np.delete(row, indices[t])
        rest = rest[np.isfinite(rest)]
        if rest.size:
            m = min(m, picked.min() - rest.max())
        out[t] = m
    return out


# ----------------------------------------------------------------------------
# Experts
# ----------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    return z / (1.0 + np.exp(-z))


# READING of gpt-oss's "swigluoai" ([SGL48763] DraftMLP commit note names it
# as an activation; no page defines it): the form gpt-oss publishes with its
# model, h = g * sigmoid(alpha * g) * (u + 1) with alpha = 1.702, on the same
# clamped pre-activations as the SwiGLU clamp below (g capped above at +limit,
# u clipped to [-limit, +limit]; gpt-oss uses limit 7).  Parity unpinned by
# the pages: its pins check this reading, not the pages.
SWIGLU_OAI_ALPHA = 1.702
ACTIVATIONS = ("swiglu", "swiglu_oai")


def swiglu(gate_pre: np.ndarray, up_pre: np.ndarray, limit: float,
           activation: str = "swiglu") -> np.ndarray:
    """SwiGLU activation with the optional clamp.

    [SGL48763] Modifications / DraftMLP commit note: gate-up and down linears
    with silu, or DeepSeek's clamped SwiGLU; [SF1073] DeepSeek-V4 family commit
    note (swiglu_limit on routed and shared experts).  READING of the clamp
    (the pages do not spell it out): the gate pre-activation is capped above at
    +limit, the up pre-activation is clipped to [-limit, +limit];
    limit = +inf means no clamp.

    activation "swiglu":     silu(g) * u
    activation "swiglu_oai": g * sigmoid(SWIGLU_OAI_ALPHA * g) * (u + 1)
    (g, u the clamped gate and up pre-activations).
    """
    if math.isinf(limit):
        g, u = gate_pre, up_pre
    else:
        g, u = np.minimum(gate_pre, limit), np.clip(up_pre, -limit, limit)
    if activation == "swiglu":
        return silu(g) * u
    if activation == "swiglu_oai":
        return g / (1.0 + np.exp(-SWIGLU_OAI_ALPHA * g)) * (u + 1.0)
    raise ValueError(activation)


def expert_mlp(rows64: np.ndarray, w_gate_up64: np.ndarray, w_down64: np.ndarray,
               limit: float, b_gate_up64=None, b_down64=None,
               activation: str = "swiglu") -> np.ndarray:
    """One expert (or the dense/shared MLP) on rows [n, H] -> [n, H], fp64.

    w_gate_up is the stacked [2I, H] matrix ([SF1073] converter commit note:
    w1 and w3 fused into gate_up_proj, w2 into down_proj).  READING: rows
    [0, I) are the gate (w1), rows [I, 2I) the up projection (w3).  The
    optional per-expert biases of the gpt-oss-style experts ([MI143]) are
    added to the pre-activations and to the output.
    """
    i2 = w_gate_up64.shape[0]
    inter = i2 // 2
    pre = rows64 @ w_gate_up64.T
    if b_gate_up64 is not None:
        pre = pre + b_gate_up64
    h = swiglu(pre[:, :inter], pre[:, inter:], limit, activation)
    y = h @ w_down64.T
    if b_down64 is not None:
        y = y + b_down64
    return y


@dataclass
class ExpertWeights:
    """One expert's weights in fp64: w_gate_up [2I, H], w_down [H, I], and the
    optional biases b_gate_up [2I], b_down [H]."""
    w_gate_up: np.ndarray
    w_down: np.ndarray
    b_gate_up: Optional[np.ndarray] = None
    b_down: Optional[np.ndarray] = None


def expert_counts(indices: np.ndarray, n_experts: int) -> np.ndarray:
    """Kept slots per expert ([SF1073] commit note on tokens_per_expert)."""
    return np.bincount(np.asarray(indices).ravel(), minlength=n_experts).astype(np.int64)


def permutation(indices: np.ndarray, n_experts: int):
    """Slots t*K+k grouped by expert, stable in slot order.

    Returns (slots [T*K], offsets [E+1]); the rows of expert e are
    slots[offsets[e]:offsets[e+1]].
    """
    flat = np.asarray(indices).ravel()
    slots = np.argsort(flat, kind="stable")
    offs = np.zeros(n_experts + 1, dtype=np.int64)
    offs[1:] = np.cumsum(expert_counts(indices, n_experts))
    return slots, offs


def routed_grouped(x64: np.ndarray, indices: np.ndarray, weights32: np.ndarray,
                   get_expert: Callable[[int], ExpertWeights], n_experts: int,
                   limit: float, activation: str = "swiglu") -> np.ndarray:
    """Weighted routed output [T, H] (fp64), expert-grouped coding.

    Slots are grouped by expert (permutation), each expert runs once on its
    rows, and each row's output is added to its token with the slot's weight,
    in k order per token ([SF1033] routing_weights row: the weights combine the
    experts' outputs).
    """
    t_count, k = indices.shape
    slots, offs = permutation(indices, n_experts)
    y_slot = np.zeros((t_count * k, x64.shape[1]), dtype=F64)
    for e in range(n_experts):
        sl = slots[offs[e]:offs[e + 1]]
        if sl.size == 0:
            continue
        w = get_expert(e)
        y_slot[sl] = expert_mlp(x64[sl // k], w.w_gate_up, w.w_down, limit,
                                w.b_gate_up, w.b_down, activation)
    out = np.zeros_like(x64)
    w64 = weights32.astype(F64)
    for kk in range(k):
        out += w64[:, kk:kk + 1] * y_slot[np.arange(t_count) * k + kk]
    return out


def routed_loop(x64: np.ndarray, indices: np.ndarray, weights32: np.ndarray,
                get_expert: Callable[[int], ExpertWeights], limit: float,
                activation: str = "swiglu") -> np.ndarray:
    """The same routed output, token by token (a second, independent coding)."""
    t_count, k = indices.shape
    out = np.zeros_like(x64)
    for t in range(t_count):
        acc = np.zeros(x64.shape[1], dtype=F64)
        for kk in range(k):
            w = get_expert(int(indices[t, kk]))
            y = expert_mlp(x64[t:t + 1], w.w_gate_up, w.w_down, limit,
                           w.b_gate_up, w.b_down, activation)[0]
            acc = acc + F64(weights32[t, kk]) * y
        out[t] = acc
    return out


def shared_expert(x64: np.ndarray, sh_gate_up64: np.ndarray, sh_down64: np.ndarray,
                  limit: float, sh_gate64: Optional[np.ndarray],
                  activation: str = "swiglu") -> np.ndarray:
    """gamma_t * SwiGLU-MLP(x_t) [T, H], fp64.

    [SGL48763] DraftMoE commit notes: the shared expert is a DraftMLP with an
    optional sigmoid gate, added to the routed sum; [SF941] "What": the
    Qwen-style block's sigmoid-gated shared expert; [SF1073] DeepSeek-V4
    family: one ungated shared expert with the same clamp.  READING: the gate
    is a bias-free H -> 1 linear, gamma = sigmoid(x . sh_gate); ungated means
    gamma = 1; route_scale does not touch the shared expert.  The layer's
    activation (and clamp) applies to the shared expert as to the routed ones.
    """
    sh = expert_mlp(x64, sh_gate_up64, sh_down64, limit, activation=activation)
    if sh_gate64 is None:
        return sh
    gamma = 1.0 / (1.0 + np.exp(-(x64 @ sh_gate64)))
    return gamma[:, None] * sh


def ffn_forward(x64, gate64, get_expert, *, n_experts, k, score_fn="softmax",
                n_group=1, topk_group=1, norm_topk_prob=True, route_scale=1.0,
                expert_bias=None, router_bias=None, limit=math.inf,
                sh_gate_up64=None, sh_down64=None, sh_gate64=None,
                coding="grouped", activation="swiglu"):
    """Whole layer forward: (RouteResult, out [T, H] fp64).

    out[t] = sum_k w[t,k] * expert_{idx[t,k]}(x_t) + gamma_t * shared(x_t).
    """
    r = route(x64, gate64, k=k, score_fn=score_fn, n_group=n_group,
              topk_group=topk_group, norm_topk_prob=norm_topk_prob,
              route_scale=route_scale, expert_bias=expert_bias,
              router_bias=router_bias)
    if coding == "grouped":
        out = routed_grouped(x64, r.indices, r.weights, get_expert, n_experts, limit, activation)
    elif coding == "loop":
        out = routed_loop(x64, r.indices, r.weights, get_expert, limit, activation)
    else:
        raise ValueError(coding)
    if sh_gate_up64 is not None:
        out = out + shared_expert(x64, sh_gate_up64, sh_down64, limit, sh_gate64, activation)
    return r, out


def token_output(x_row64, indices_row, weights_row32, get_expert, limit,
                 sh_gate_up64=None, sh_down64=None, sh_gate64=None,
                 activation="swiglu") -> np.ndarray:
    """One token's output row [H] (fp64) given its routing; for sampled checks
    at sizes where the whole layer is too large to evaluate on the CPU."""
    x1 = np.asarray(x_row64, dtype=F64)[None, :]
    acc = np.zeros(x1.shape[1], dtype=F64)
    for kk in range(len(indices_row)):
        w = get_expert(int(indices_row[kk]))
        acc = acc + F64(weights_row32[kk]) * expert_mlp(
            x1, w.w_gate_up, w.w_down, limit, w.b_gate_up, w.b_down, activation)[0]
    if sh_gate_up64 is not None:
        acc = acc + shared_expert(x1, sh_gate_up64, sh_down64, limit, sh_gate64, activation)[0]
    return acc


# ----------------------------------------------------------------------------
# Load-balancing state ([SF1073] commit notes on tokens_per_expert, on
# MoEBalancing's moe/step_balance and on update_expert_bias)
# ----------------------------------------------------------------------------
def masked_expert_counts(indices: np.ndarray, n_experts: int,
                         token_mask: Optional[np.ndarray] = None) -> np.ndarray:
    """Kept slots per expert, int64 [E].

    [SF1073] commit note on tokens_per_expert: each training forward adds its
    kept slots, those of tokens that moe_token_mask keeps, to an int64 count
    per expert.  READING: the mask is one flag per token (the kept-block mask
    expanded to draft tokens, per the note on moe_token_mask) and a kept token
    contributes all K of its slots; no mask keeps every token.
    """
    idx = np.asarray(indices)
    counts = np.zeros(n_experts, dtype=np.int64)
    for t in range(idx.shape[0]):
        if token_mask is not None and not bool(token_mask[t]):
            continue
        for k in range(idx.shape[1]):
            counts[int(idx[t, k])] += 1
    return counts


def step_balance(counts: np.ndarray) -> float:
    """moe/step_balance of pooled counts, as fp32.

    [SF1073] commit note on MoEBalancing: 1 when the load is uniform, E / K
    when it has collapsed onto K experts.  READING: the largest count over the
    mean count, E * max(c) / sum(c) (the only plain ratio with both stated
    values); evaluated in fp64, rounded once to fp32.  READING: with no kept
    slot the load counts as uniform, 1.
    """
    c = np.asarray(counts, dtype=np.int64)
    total = int(c.sum())
    if total == 0:
        return float(F32(1.0))
    return float(F32(F64(c.size) * F64(int(c.max())) / F64(total)))


def update_expert_bias(expert_bias32: np.ndarray, counts: np.ndarray, rate: float) -> np.ndarray:
    """One DeepSeek-V3 sign step of the selection-only expert bias, fp32 [E].

    [SF1073] commit note on update_expert_bias: one sign step with a
    zero-mean delta, fed the step's pooled kept-slot counts; rate 0 keeps the
    bias fixed.  The step raises the bias of experts below the mean load and
    lowers it for those above: s_e = sign(mean(c) - c_e), decided exactly on
    integers as sign(sum(c) - E * c_e).  READING of "zero-mean": the delta is
    rate * (s_e - mean(s)), with mean(s) = sum(s) / E; fp32 arithmetic in this
    order: m = f32(sum s) / f32(E); d_e = f32(rate) * (f32(s_e) - m);
    bias_e + d_e.
    """
    b = np.asarray(expert_bias32, dtype=F32).copy()
    if rate == 0.0:
        return b
    c = np.asarray(counts, dtype=np.int64)
    n = c.size
    total = int(c.sum())
    s = np.array([(total > n * int(ce)) - (total < n * int(ce)) for ce in c], dtype=np.int64)
    m = F32(F32(int(s.sum())) / F32(n))
    r = F32(rate)
    for e in range(n):
        d = F32(r * F32(F32(int(s[e])) - m))
        b[e] = F32(b[e] + d)
    return b


# ----------------------------------------------------------------------------
# Backward of the layer ([SF1033] "Router" section: forward returns scores,
# indices, weights and the MoE FFN trains with grouped GEMMs; [SF1073] commit
# note on the V4.1 port: the forward output and every gradient are compared;
# the expert bias shifts the picks, never the weights)
# ----------------------------------------------------------------------------
@dataclass
class LayerGrads:
    """Gradients of sum(out * dout) with respect to every input, fp64."""
    dx: np.ndarray                      # [T, H]
    dgate: np.ndarray                   # [E, H]
    drouter_bias: Optional[np.ndarray]  # [E] (logit-bias variant only)
    dw_gate_up: dict                    # e -> [2I, H], experts with slots only
    dw_down: dict                       # e -> [H, I]
    db_gate_up: dict                    # e -> [2I] (experts with linear biases)
    db_down: dict                       # e -> [H]
    dsh_gate_up: Optional[np.ndarray]   # [2Is, H]
    dsh_down: Optional[np.ndarray]      # [H, Is]
    dsh_gate: Optional[np.ndarray]      # [H]
    dweights: Optional[np.ndarray] = None  # [T, K]: d of the routing weights, dout_t . y_k


def swiglu_backward(gate_pre: np.ndarray, up_pre: np.ndarray, limit: float,
                    dh: np.ndarray, activation: str = "swiglu"):
    """(d gate_pre, d up_pre) of h = act(min(g, L), clip(u, -L, L)).

    "swiglu": act = silu(g) u, silu'(z) = sigma(z) * (1 + z * (1 - sigma(z)));
    "swiglu_oai": act = g sigma(a g) (u + 1), d/dg = sigma(a g) (1 + a g
    (1 - sigma(a g))) (u + 1), d/du = g sigma(a g).  READING: where the clamp
    binds the gradient is cut; on the boundary itself (g = L, u = +-L) it
    passes, as for a clamp whose gradient mask is inclusive.
    """
    g = np.asarray(gate_pre, dtype=F64)
    u = np.asarray(up_pre, dtype=F64)
    if math.isinf(limit):
        gc, uc = g, u
        g_pass = np.ones_like(g, dtype=bool)
        u_pass = np.ones_like(u, dtype=bool)
    else:
        gc, uc = np.minimum(g, limit), np.clip(u, -limit, limit)
        g_pass = g <= limit
        u_pass = (u >= -limit) & (u <= limit)
    a = 1.0 if activation == "swiglu" else SWIGLU_OAI_ALPHA
    if activation not in ACTIVATIONS:
        raise ValueError(activation)
    sig = 1.0 / (1.0 + np.exp(-a * gc))
    glu = gc * sig
    dglu = sig * (1.0 + a * gc * (1.0 - sig))
    lin = uc if activation == "swiglu" else uc + 1.0
    dg = np.where(g_pass, dh * lin * dglu, 0.0)
    du = np.where(u_pass, dh * glu, 0.0)
    return dg, du


def score_backward(logits64: np.ndarray, scores64: np.ndarray, dscores: np.ndarray,
                   fn: str) -> np.ndarray:
    """d logits [E] of one token's scores [E] (fp64 values).

    softmax: ds -> s * (ds - sum(ds * s)); sigmoid: ds * s * (1 - s);
    sqrt(softplus(l)): ds * sigma(l) / (2 s).
    """
    l = np.asarray(logits64, dtype=F64)
    s = np.asarray(scores64, dtype=F64)
    ds = np.asarray(dscores, dtype=F64)
    if fn == "softmax":
        return s * (ds - np.dot(ds, s))
    if fn == "sigmoid":
        return ds * s * (1.0 - s)
    if fn == "sqrtsoftplus":
        return ds * (1.0 / (1.0 + np.exp(-l))) / (2.0 * s)
    raise ValueError(fn)


def weights_backward(picked64: np.ndarray, dweights: np.ndarray, norm_topk_prob: bool,
                     route_scale: float, eps: float = float(RENORM_EPS)) -> np.ndarray:
    """d picked scores [K] of w_k = rs * s_k / (sum_j s_j + eps) (renormalised)
    or w_k = rs * s_k."""
    s = np.asarray(picked64, dtype=F64)
    dw = np.asarray(dweights, dtype=F64)
    rs = float(route_scale)
    if not norm_topk_prob:
        return rs * dw
    d = s.sum() + eps
    return rs * dw / d - rs * np.dot(dw, s) / (d * d)


def _scores64(x, gate, router_bias, score_fn):
    """fp64 logits [T, E] and scores [T, E], not rounded: the point at which
    the backward differentiates (the score functions of route())."""
    logits = x @ gate.T
    if router_bias is not None:
        logits = logits + np.asarray(router_bias, dtype=F64)
    if score_fn == "softmax":
        z = np.exp(logits - logits.max(axis=-1, keepdims=True))
        scores = z / z.sum(axis=-1, keepdims=True)
    elif score_fn == "sigmoid":
        scores = 1.0 / (1.0 + np.exp(-logits))
    else:
        scores = np.sqrt(np.maximum(logits, 0.0) + np.log1p(np.exp(-np.abs(logits))))
    return logits, scores


def _picked_weights(picked, norm_topk_prob, route_scale):
    """Routing weights of the picked scores (last axis: the k slots), as the
    forward forms them: renormalised with the +1e-20 guard, times route_scale."""
    if norm_topk_prob:
        return route_scale * picked / (picked.sum(axis=-1, keepdims=True) + float(RENORM_EPS))
    return route_scale * picked


def backward_routing_weights(x64, gate64, indices, *, score_fn="softmax", norm_topk_prob=True,
                             route_scale=1.0, router_bias=None) -> np.ndarray:
    """fp64 routing weights [T, K] at the given selection: the weights at
    which ffn_backward differentiates the experts (fp64 scores of fp64 logits,
    picked, renormalised and scaled as the forward does)."""
    _, scores = _scores64(np.asarray(x64, dtype=F64), np.asarray(gate64, dtype=F64), router_bias, score_fn)
    picked = np.take_along_axis(scores, np.asarray(indices, dtype=np.int64), axis=1)
    return _picked_weights(picked, norm_topk_prob, route_scale)


def expert_grad_rows(x64, dout64, tokens, weights, ew: "ExpertWeights", cols, *,
                     limit=math.inf, activation="swiglu"):
    """Sampled entries of one routed expert's weight gradients.

    [SF1073] V4.1 port note (forward and every gradient compared).  The
    expert adds w * y to the output of each token routed to it (token ids
    `tokens`, routing weights `weights`), with pre = W_gu x (+ b_gu),
    h_j = act(pre_j, pre_{I+j}), y = W_d h (+ b_d).  Differentiating:
    dy = w dout, (dh)_j = W_d[:, j] . dy, the SwiGLU derivative gives
    d pre_j and d pre_{I+j}, and
        dW_gu[j, :]   = sum over the tokens of d pre_j   x,
        dW_gu[I+j, :] = sum over the tokens of d pre_{I+j} x,
        dW_d[:, j]    = sum over the tokens of h_j dy.
    Column j of h needs only rows j and I + j of W_gu and column j of W_d,
    so these entries cost a few dot products per token, at any layer size.
    Returns (dW_gu rows [2, len(cols), H]: the gate rows, then the up rows;
    dW_d columns [H, len(cols)])."""
    tokens = np.asarray(tokens, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    x = np.asarray(x64, dtype=F64)[tokens]
    dy = np.asarray(weights, dtype=F64)[:, None] * np.asarray(dout64, dtype=F64)[tokens]
    wgu = np.asarray(ew.w_gate_up, dtype=F64)
    wd = np.asarray(ew.w_down, dtype=F64)
    inter = wgu.shape[0] // 2
    pg = x @ wgu[cols].T
    pu = x @ wgu[inter + cols].T
    if ew.b_gate_up is not None:
        b = np.asarray(ew.b_gate_up, dtype=F64)
        pg, pu = pg + b[cols], pu + b[inter + cols]
    h = swiglu(pg, pu, limit, activation)
    dh = dy @ wd[:, cols]
    dg, du = swiglu_backward(pg, pu, limit, dh, activation)
    return np.stack([dg.T @ x, du.T @ x]), dy.T @ h


def ffn_backward(x64, gate64, get_expert, dout64, *, n_experts, k, score_fn="softmax",
                 n_group=1, topk_group=1, norm_topk_prob=True, route_scale=1.0,
                 expert_bias=None, router_bias=None, limit=math.inf,
                 sh_gate_up64=None, sh_down64=None, sh_gate64=None,
                 activation="swiglu") -> LayerGrads:
    """Gradients of the layer at (x, weights) for the output gradient dout.

    The selection (indices) is the forward's (route(), fp32 decisions) and is
    held fixed: it is piecewise constant, and the expert bias that shifts it
    gets no gradient.  Everything else is differentiated exactly in fp64 at
    fp64 values (logits, scores, weights and pre-activations are not rounded
    here).  Steps, the forward's in reverse: combine -> routed experts (down,
    SwiGLU, gate_up) and shared expert (with its sigmoid gate) -> routing
    weights -> scores -> logits -> gate and x.
    """
    x = np.asarray(x64, dtype=F64)
    gate = np.asarray(gate64, dtype=F64)
    dout = np.asarray(dout64, dtype=F64)
    r = route(x, gate, k=k, score_fn=score_fn, n_group=n_group, topk_group=topk_group,
              norm_topk_prob=norm_topk_prob, route_scale=route_scale,
              expert_bias=expert_bias, router_bias=router_bias)
    idx = r.indices
    t_count, h_dim = x.shape
    logits, scores = _scores64(x, gate, router_bias, score_fn)

    dx = np.zeros_like(x)
    dgate = np.zeros_like(gate)
    drb = np.zeros(n_experts) if router_bias is not None else None
    dwgu, dwd, dbgu, dbd = {}, {}, {}, {}
    dweights_all = np.zeros((t_count, k))
    has_sh = sh_gate_up64 is not None
    if has_sh:
        wsgu = np.asarray(sh_gate_up64, dtype=F64)
        wsd = np.asarray(sh_down64, dtype=F64)
        dsgu, dsd = np.zeros_like(wsgu), np.zeros_like(wsd)
        dsg = np.zeros(h_dim) if sh_gate64 is not None else None
    for t in range(t_count):
        xt, dt = x[t], dout[t]
        picked = scores[t, idx[t]]
        w = _picked_weights(picked, norm_topk_prob, route_scale)
        dweights = np.zeros(k)
        for kk in range(k):
            e = int(idx[t, kk])
            ew = get_expert(e)
            wgu, wd = np.asarray(ew.w_gate_up, dtype=F64), np.asarray(ew.w_down, dtype=F64)
            inter = wgu.shape[0] // 2
            pre = wgu @ xt
            if ew.b_gate_up is not None:
                pre = pre + ew.b_gate_up
            h = swiglu(pre[:inter], pre[inter:], limit, activation)
            y = wd @ h
            if ew.b_down is not None:
                y = y + ew.b_down
            # combine: out_t += w_k * y_k
            dweights[kk] = np.dot(dt, y)
            dy = w[kk] * dt
            # down: y = Wd h (+ b)
            dh = wd.T @ dy
            dwd[e] = dwd.get(e, 0.0) + np.outer(dy, h)
            if ew.b_down is not None:
                dbd[e] = dbd.get(e, 0.0) + dy
            # SwiGLU and gate_up: pre = Wgu x (+ b)
            dg, du = swiglu_backward(pre[:inter], pre[inter:], limit, dh, activation)
            dpre = np.concatenate([dg, du])
            dwgu[e] = dwgu.get(e, 0.0) + np.outer(dpre, xt)
            if ew.b_gate_up is not None:
                dbgu[e] = dbgu.get(e, 0.0) + dpre
            dx[t] += wgu.T @ dpre
        if has_sh:
            inter_s = wsgu.shape[0] // 2
            pre_s = wsgu @ xt
            h_s = swiglu(pre_s[:inter_s], pre_s[inter_s:], limit, activation)
            sh = wsd @ h_s
            gam = 1.0 / (1.0 + np.exp(-np.dot(xt, sh_gate64))) if sh_gate64 is not None else 1.0
            dsh = gam * dt
            dh_s = wsd.T @ dsh
            dsd += np.outer(dsh, h_s)
            dg_s, du_s = swiglu_backward(pre_s[:inter_s], pre_s[inter_s:], limit, dh_s, activation)
            dpre_s = np.concatenate([dg_s, du_s])
            dsgu += np.outer(dpre_s, xt)
            dx[t] += wsgu.T @ dpre_s
            if sh_gate64 is not None:
                dz = np.dot(dt, sh) * gam * (1.0 - gam)
                dx[t] += dz * np.asarray(sh_gate64, dtype=F64)
                dsg += dz * xt
        dweights_all[t] = dweights
        # routing weights -> scores -> logits
        ds = np.zeros(n_experts)
        ds[idx[t]] = weights_backward(picked, dweights, norm_topk_prob, route_scale)
        dl = score_backward(logits[t], scores[t], ds, score_fn)
        if drb is not None:
            drb += dl
        dgate += np.outer(dl, xt)
        dx[t] += gate.T @ dl
    return LayerGrads(dx, dgate, drb, dwgu, dwd, dbgu, dbd,
                      dsgu if has_sh else None, dsd if has_sh else None,
                      dsg if has_sh and sh_gate64 is not None else None, dweights_all)
