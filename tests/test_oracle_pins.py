"""Pins of the CPU oracle against things other than itself.

Each test checks one oracle function against brute force, a closed form, a
library routine or an invariant the pages state, chosen so that a plausible
slip (a dropped term, a wrong sign or index, a transposed operand, a wrong
tie rule) fails one of them.  CPU only.

Pages cited: [SF1033] SpecForge PR #1033 "MoE FFN for DFlash-family drafts:
the module" (Router table; commit note on the 1e-20 epsilon); [SF1073]
SpecForge PR #1073 "MoE drafts: DeepSeek-V4.1's own DSpark draft (stacked on
#1035)" (commit notes on the expert bias, on select receiving shifted scores,
on the DeepSeek-V4 family and on the V4.1 converter's FP4 packing); [MI143]
MoE-Infinity PR #143 (commit note on the resident gpt-oss MXFP4 experts);
[SGL48763] sglang PR #48763 "[Feat] dflash: Serve MoE FFN drafts for DFlash
and DSpark" (DraftMLP / DraftMoE commit notes).
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import moe_oracle as O

F32 = np.float32
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def ulp32(x):
    return np.spacing(np.abs(np.asarray(x, dtype=F32))).astype(np.float64)


# ----------------------------------------------------------------------------
# number formats
# ----------------------------------------------------------------------------

def test_bf16_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x3F81, 0x0001, 0x7F7F, 0x4049], dtype=np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, 1.0 + 2.0 ** -7, 2.0 ** -133,
            (2 - 2.0 ** -7) * 2.0 ** 127, 3.140625]
    got = O.bf16_to_f64(bits)
    assert list(got) == want
    assert math.copysign(1.0, got[3]) == -1.0


def test_bf16_matches_torch_widening():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 65536, size=4096, dtype=np.int64).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]           # drop inf/nan patterns
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.bf16_to_f64(bits), t)


def _golden_e2m1():
    with open(os.path.join(GOLDEN, "e2m1_table.json")) as f:
        return json.load(f)


def test_e2m1_exhaustive_table():
    g = _golden_e2m1()
    codes = np.arange(16)
    assert list(O.e2m1_to_f64(codes)) == g["values"]


def test_e8m0_scales():
    s = np.array([0, 1, 124, 125, 126, 127, 128, 254, 255])
    got = O.e8m0_to_f64(s)
    want = [2.0 ** -127, 2.0 ** -126, 0.125, 0.25, 0.5, 1.0, 2.0, 2.0 ** 127]
    assert list(got[:-1]) == want
    assert np.isnan(got[-1])


def test_mxfp4_nibble_order_and_scale_blocks():
    # one output row, 64 inputs: byte j holds inputs 2j (low nibble) and 2j+1 (high)
    codes = np.zeros((1, 32), dtype=np.uint8)
    codes[0, 0] = 0x21          # input 0 <- code 1 (0.5), input 1 <- code 2 (1.0)
    codes[0, 16] = 0xF7         # input 32 <- code 7 (6.0), input 33 <- code 15 (-6.0)
    scales = np.array([[127, 129]], dtype=np.uint8)   # inputs 0..31 x1, 32..63 x4
    w = O.mxfp4_dequant(codes, scales)
    assert w.shape == (1, 64)
    assert w[0, 0] == 0.5 and w[0, 1] == 1.0
    assert w[0, 32] == 24.0 and w[0, 33] == -24.0
    assert np.count_nonzero(w) == 4


def _encode_e2m1(v):
    """Independent encoder: value in the E2M1 set -> code (lookup by value)."""
    table = {0.5: 1, 1.0: 2, 1.5: 3, 2.0: 4, 3.0: 5, 4.0: 6, 6.0: 7}
    if v == 0:
        return 0
    return table[abs(v)] | (8 if v < 0 else 0)


def test_mxfp4_pack_roundtrip_is_exact():
    rng = np.random.default_rng(7)
    n, kin = 5, 96
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    base = rng.choice(mags, size=(n, kin)) * rng.choice([-1.0, 1.0], size=(n, kin))
    sc = rng.integers(120, 135, size=(n, kin // 32))
    values = base * np.repeat(2.0 ** (sc - 127.0), 32, axis=1)
    codes = np.zeros((n, kin // 2), dtype=np.uint8)
    for r in range(n):
        for k in range(kin):
            c = _encode_e2m1(base[r, k])
            codes[r, k // 2] |= (c << 4) if (k % 2) else c
    got = O.mxfp4_dequant(codes, sc.astype(np.uint8))
    assert np.array_equal(got, values)
    # every value is exact in bf16 as well: widening its bf16 pattern is identity
    b = torch.from_numpy(values).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(b, values)


# ----------------------------------------------------------------------------
# router logits and scores
# ----------------------------------------------------------------------------

def test_router_logits_are_the_rounded_exact_dot():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((6, 40)).astype(F32).astype(np.float64)
    g = (0.02 * rng.standard_normal((5, 40))).astype(F32).astype(np.float64)
    got = O.router_logits(x, g)
    for t in range(6):
        for e in range(5):
            exact = math.fsum(float(a) * float(b) for a, b in zip(x[t], g[e]))
            # BLAS fp64 sum differs from the exact sum by far less than an fp32 ulp
            assert abs(float(got[t, e]) - exact) <= 0.5 * float(ulp32(exact)) * 1.0001
    # orientation: logits[t, e] uses row e of the gate
    e1 = np.zeros((1, 40)); e1[0, 3] = 1.0
    gg = np.zeros((5, 40)); gg[2, 3] = 2.0
    assert O.router_logits(e1, gg)[0].tolist() == [0, 0, 2.0, 0, 0]


def test_router_bias_adds_after_rounding():
    x = np.ones((1, 4)); g = np.full((3, 4), 0.25)
    rb = np.array([0.5, -1.0, 0.0], dtype=F32)
    assert O.router_logits(x, g, rb)[0].tolist() == [1.5, 0.0, 1.0]


def test_score_closed_forms():
    z = np.zeros((1, 8), dtype=F32)
    assert np.all(O.score(z, "softmax") == F32(0.125))
    assert np.all(O.score(z, "sigmoid") == F32(0.5))
    assert np.all(O.score(z, "sqrtsoftplus") == F32(math.sqrt(math.log(2.0))))


def test_sigmoid_symmetry():
    rng = np.random.default_rng(4)
    l = rng.uniform(-6, 6, size=(1, 512)).astype(F32)
    a = O.score(l, "sigmoid").astype(np.float64)
    b = O.score(-l, "sigmoid").astype(np.float64)
    assert np.all(np.abs(a + b - 1.0) <= ulp32(np.maximum(a, b)))


@pytest.mark.parametrize("fn", ["softmax", "sigmoid", "sqrtsoftplus"])
def test_scores_match_torch(fn):
    rng = np.random.default_rng(5)
    l = (1.5 * rng.standard_normal((16, 64))).astype(F32)
    lt = torch.from_numpy(l).to(torch.float64)
    if fn == "softmax":
        ref = torch.softmax(lt, dim=-1)
    elif fn == "sigmoid":
        ref = torch.sigmoid(lt)
    else:
        ref = torch.sqrt(F.softplus(lt, threshold=1000.0))
    ref = ref.to(torch.float32).numpy()
    got = O.score(l, fn)
    assert np.all(np.abs(got.astype(np.float64) - ref) <= ulp32(ref))
    if fn == "softmax":
        assert np.all(got >= 0) and np.all(got <= 1)
        assert np.allclose(got.sum(-1), 1.0, atol=64 * 2.0 ** -24)


def test_sqrtsoftplus_large_and_small():
    l = np.array([[40.0, -40.0, 0.0]], dtype=F32)
    s = O.score(l, "sqrtsoftplus")[0].astype(np.float64)
    assert s[0] == F32(math.sqrt(40.0))
    assert abs(s[1] - math.sqrt(math.exp(-40.0))) <= 1e-6 * math.sqrt(math.exp(-40.0))


# ----------------------------------------------------------------------------
# select
# ----------------------------------------------------------------------------

def _order_key(v, i):
    return (-float(v), int(i))


def brute_topk(values, k):
    """The unique K-subset that dominates every outsider under the order
    (value descending, index ascending), listed in that order."""
    e = len(values)
    found = []
    for sub in itertools.combinations(range(e), k):
        rest = [j for j in range(e) if j not in sub]
        if all(_order_key(values[i], i) < _order_key(values[j], j) for i in sub for j in rest):
            found.append(sub)
    assert len(found) == 1
    return sorted(found[0], key=lambda i: _order_key(values[i], i))


def brute_group_topk(values, k, n_group, topk_group):
    e = len(values)
    size = e // n_group
    gscore = []
    for g in range(n_group):
        mem = values[g * size:(g + 1) * size]
        best = max(F32(mem[i] + mem[j]) for i in range(size) for j in range(size) if i < j)
        gscore.append(best)
    keep = brute_topk(np.array(gscore, dtype=F32), topk_group)
    allowed = sorted(i for g in keep for i in range(g * size, (g + 1) * size))
    sub = brute_topk(values[allowed], k)
    return [allowed[i] for i in sub]


def test_select_plain_matches_brute_force_with_ties():
    rng = np.random.default_rng(11)
    for trial in range(300):
        e = int(rng.integers(2, 11))
        k = int(rng.integers(1, min(e, 3) + 1))
        vals = rng.choice(np.array([0.0, 0.25, 0.5, 0.75], dtype=F32), size=e)
        got = O.select(vals[None, :], k)[0].tolist()
        assert got == brute_topk(vals, k), (vals, k)


def test_select_group_limited_matches_brute_force():
    rng = np.random.default_rng(12)
    for trial in range(300):
        n_group = int(rng.choice([2, 3, 4]))
        size = int(rng.choice([2, 3]))
        e = n_group * size
        topk_group = int(rng.integers(1, n_group + 1))
        k = int(rng.integers(1, min(3, topk_group * size) + 1))
        vals = rng.choice(np.array([-0.5, 0.0, 0.125, 0.25, 0.5], dtype=F32), size=e)
        got = O.select(vals[None, :], k, n_group, topk_group)[0].tolist()
        assert got == brute_group_topk(vals, k, n_group, topk_group), (vals, k, n_group, topk_group)


def test_group_limited_reduces_to_plain():
    rng = np.random.default_rng(13)
    c = rng.standard_normal((20, 32)).astype(F32)
    plain = O.select(c, 6)
    assert np.array_equal(O.select(c, 6, n_group=1, topk_group=1), plain)
    assert np.array_equal(O.select(c, 6, n_group=8, topk_group=8), plain)


def test_all_ties_pick_lowest_ids_and_equal_weights():
    # a zero gate makes every logit 0: every score ties
    x = np.ones((3, 16)); g = np.zeros((8, 16))
    for fn in ("softmax", "sigmoid", "sqrtsoftplus"):
        r = O.route(x, g, k=4, score_fn=fn, route_scale=2.5)
        assert np.all(r.indices == np.arange(4))
        assert np.all(r.weights == F32(2.5 / 4))


# ----------------------------------------------------------------------------
# expert bias ([SF1073]: selection only, never the weights)
# ----------------------------------------------------------------------------

def test_bias_moves_selection_not_weights():
    rng = np.random.default_rng(21)
    x = rng.standard_normal((10, 32)); g = 0.1 * rng.standard_normal((16, 32))
    base = O.route(x, g, k=3)
    bias = np.zeros(16, dtype=F32); bias[[5, 9, 14]] = 10.0    # forces 5, 9, 14
    r = O.route(x, g, k=3, expert_bias=bias)
    assert np.all(np.sort(r.indices, axis=1) == [5, 9, 14])
    assert np.array_equal(r.scores, base.scores)              # scores unshifted
    # weights are the renormalised UNSHIFTED scores of the forced experts
    for t in range(10):
        s = base.scores[t, r.indices[t]]
        tot = F32(F32(F32(s[0] + s[1]) + s[2]) + O.RENORM_EPS)
        assert np.array_equal(r.weights[t], (s / tot).astype(F32))


def test_bias_that_keeps_selection_keeps_weights_bitwise():
    rng = np.random.default_rng(22)
    x = rng.standard_normal((12, 32)); g = 0.1 * rng.standard_normal((16, 32))
    base = O.route(x, g, k=4)
    tiny = (1e-9 * rng.standard_normal(16)).astype(F32)
    r = O.route(x, g, k=4, expert_bias=tiny)
    same = np.all(np.sort(r.indices, 1) == np.sort(base.indices, 1), axis=1)
    assert same.sum() >= 10
    for t in np.nonzero(same)[0]:
        order = np.argsort(base.indices[t])
        order2 = np.argsort(r.indices[t])
        assert np.array_equal(base.weights[t][order], r.weights[t][order2])


def test_uniform_bias_shift_changes_nothing():
    # values on a 2^-10 grid keep every fp32 sum exact, so a common shift is exact
    rng = np.random.default_rng(23)
    s = (rng.integers(0, 1024, size=(40, 16)) / 1024.0).astype(F32)
    b = (rng.integers(-64, 64, size=16) / 1024.0).astype(F32)
    c1 = O.choice(s, b)
    c2 = O.choice(s, (b + F32(0.5)).astype(F32))
    assert np.array_equal(O.select(c1, 4), O.select(c2, 4))
    assert np.array_equal(O.select(c1, 4, 4, 2), O.select(c2, 4, 4, 2))


# ----------------------------------------------------------------------------
# routing_weights
# ----------------------------------------------------------------------------

def test_renormalised_softmax_weights_sum_to_route_scale():
    rng = np.random.default_rng(31)
    x = rng.standard_normal((50, 64)); g = 0.05 * rng.standard_normal((32, 64))
    for rs in (1.0, 2.5):
        r = O.route(x, g, k=4, route_scale=rs)
        tot = r.weights.astype(np.float64).sum(1)
        assert np.all(np.abs(tot - rs) <= 4 * ulp32(rs) * 2)


def test_eps_is_bitwise_noop_for_softmax():
    # [SF1033] epsilon note: for softmax the top-k sum is at least K/E, so the
    # 1e-20 guard changes no bit of the fp32 weights.
    rng = np.random.default_rng(32)
    x = rng.standard_normal((64, 64)); g = 0.1 * rng.standard_normal((512, 64))
    lg = O.router_logits(x, g)
    s = O.score(lg, "softmax")
    idx = O.select(s, 10)
    a = O.routing_weights(s, idx, True, 1.0)
    b = O.routing_weights(s, idx, True, 1.0, eps=0.0)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_top1_renormalised_weight_is_exactly_route_scale():
    rng = np.random.default_rng(33)
    x = rng.standard_normal((30, 32)); g = 0.1 * rng.standard_normal((8, 32))
    assert np.all(O.route(x, g, k=1).weights == F32(1.0))
    assert np.all(O.route(x, g, k=1, route_scale=1.5).weights == F32(1.5))


def test_eps_guards_sigmoid_underflow():
    # every sigmoid score underflows to 0: weights must be 0, not NaN
    x = np.ones((2, 4)); g = np.full((8, 4), -60.0)
    r = O.route(x, g, k=2, score_fn="sigmoid")
    assert np.all(r.scores == 0) and np.all(r.weights == 0)
    s = r.scores
    with np.errstate(invalid="ignore"):
        no_eps = O.routing_weights(s, r.indices, True, 1.0, eps=0.0)
    assert np.all(np.isnan(no_eps))


def test_no_renorm_is_scaled_score():
    rng = np.random.default_rng(34)
    x = rng.standard_normal((5, 16)); g = 0.2 * rng.standard_normal((8, 16))
    r = O.route(x, g, k=2, score_fn="sigmoid", norm_topk_prob=False, route_scale=2.5)
    for t in range(5):
        assert np.array_equal(r.weights[t], (r.scores[t, r.indices[t]] * F32(2.5)).astype(F32))


def test_softmax_over_selected_logits_agrees():
    # gpt-oss-style coding: top-k on logits, softmax over the K picks
    rng = np.random.default_rng(35)
    x = rng.standard_normal((200, 64)); g = 0.05 * rng.standard_normal((32, 64))
    r = O.route(x, g, k=4)
    lt = torch.from_numpy(r.logits.astype(np.float64))
    top = torch.topk(lt, 4, dim=-1)
    w_alt = torch.softmax(top.values, dim=-1).numpy()
    margin = O.selection_margins(r.choice, r.indices)
    ok = margin > 1e-6
    assert ok.sum() > 190
    assert np.array_equal(top.indices.numpy()[ok], r.indices[ok])
    assert np.max(np.abs(w_alt[ok] - r.weights[ok])) <= 1e-6


# ----------------------------------------------------------------------------
# counts and permutation
# ----------------------------------------------------------------------------

def test_permutation_invariants():
    rng = np.random.default_rng(41)
    idx = np.stack([rng.permutation(12)[:3] for _ in range(37)]).astype(np.int32)
    cnt = O.expert_counts(idx, 12)
    assert cnt.sum() == idx.size
    slots, offs = O.permutation(idx, 12)
    assert sorted(slots.tolist()) == list(range(idx.size))
    flat = idx.ravel()
    for e in range(12):
        seg = slots[offs[e]:offs[e + 1]]
        assert np.all(flat[seg] == e) and len(seg) == cnt[e]
        assert np.all(np.diff(seg) > 0)     # stable: slot order inside an expert


# ----------------------------------------------------------------------------
# experts
# ----------------------------------------------------------------------------

def _rand_experts(rng, e, h, i, with_bias=False):
    ws = []
    for _ in range(e):
        ws.append(O.ExpertWeights(
            0.3 * rng.standard_normal((2 * i, h)), 0.3 * rng.standard_normal((h, i)),
            0.1 * rng.standard_normal(2 * i) if with_bias else None,
            0.1 * rng.standard_normal(h) if with_bias else None))
    return ws


def _act_scalar(g, u, limit, activation):
    """One SwiGLU element by scalar math.  swiglu_oai takes the logistic
    function in its tanh form, sigma(z) = (1 + tanh(z / 2)) / 2, a route
    independent of the oracle's 1 / (1 + exp(-z))."""
    if limit != math.inf:
        g = min(g, limit); u = max(-limit, min(limit, u))
    if activation == "swiglu_oai":
        return g * 0.5 * (1.0 + math.tanh(0.851 * g)) * (u + 1.0)     # 0.851 = 1.702 / 2
    return g / (1.0 + math.exp(-g)) * u


def _pure_python_forward(x, idx, w, experts, limit, shared=None, activation="swiglu"):
    """Brute force with scalar loops only (tiny sizes)."""
    t_count, h = x.shape
    out = [[0.0] * h for _ in range(t_count)]
    for t in range(t_count):
        for kk in range(idx.shape[1]):
            ex = experts[int(idx[t, kk])]
            inter = ex.w_gate_up.shape[0] // 2
            hv = []
            for j in range(inter):
                g = sum(x[t, c] * ex.w_gate_up[j, c] for c in range(h))
                u = sum(x[t, c] * ex.w_gate_up[inter + j, c] for c in range(h))
                if ex.b_gate_up is not None:
                    g += ex.b_gate_up[j]; u += ex.b_gate_up[inter + j]
                hv.append(_act_scalar(g, u, limit, activation))
            for n in range(h):
                y = sum(hv[j] * ex.w_down[n, j] for j in range(inter))
                if ex.b_down is not None:
                    y += ex.b_down[n]
                out[t][n] += float(w[t, kk]) * y
        if shared is not None:
            gu, dn, gv = shared
            inter = gu.shape[0] // 2
            hv = []
            for j in range(inter):
                g = sum(x[t, c] * gu[j, c] for c in range(h))
                u = sum(x[t, c] * gu[inter + j, c] for c in range(h))
                hv.append(_act_scalar(g, u, limit, activation))
            gamma = 1.0 if gv is None else 1.0 / (1.0 + math.exp(-sum(x[t, c] * gv[c] for c in range(h))))
            for n in range(h):
                out[t][n] += gamma * sum(hv[j] * dn[n, j] for j in range(inter))
    return np.array(out)


@pytest.mark.parametrize("limit,bias,shared,gated,activation", [
    (math.inf, False, False, False, "swiglu"), (0.7, False, True, True, "swiglu"),
    (0.7, True, False, False, "swiglu"), (math.inf, False, True, False, "swiglu"),
    (0.7, True, True, True, "swiglu_oai"), (math.inf, False, True, False, "swiglu_oai")])
def test_forward_matches_pure_python(limit, bias, shared, gated, activation):
    rng = np.random.default_rng(51)
    t_count, h, i, e, k = 5, 6, 3, 4, 2
    x = rng.standard_normal((t_count, h))
    gate = rng.standard_normal((e, h))
    experts = _rand_experts(rng, e, h, i, bias)
    sh = None
    kw = {}
    if shared:
        sh = (0.3 * rng.standard_normal((4, h)), 0.3 * rng.standard_normal((h, 2)),
              0.3 * rng.standard_normal(h) if gated else None)
        kw = dict(sh_gate_up64=sh[0], sh_down64=sh[1], sh_gate64=sh[2])
    r, out = O.ffn_forward(x, gate, lambda j: experts[j], n_experts=e, k=k,
                           limit=limit, activation=activation, **kw)
    ref = _pure_python_forward(x, r.indices, r.weights, experts, limit, sh, activation)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_grouped_and_loop_codings_agree():
    rng = np.random.default_rng(52)
    t_count, h, i, e, k = 40, 32, 16, 12, 3
    x = rng.standard_normal((t_count, h))
    gate = 0.2 * rng.standard_normal((e, h))
    experts = _rand_experts(rng, e, h, i, True)
    bias = (0.05 * rng.standard_normal(e)).astype(F32)
    kw = dict(n_experts=e, k=k, score_fn="sigmoid", n_group=4, topk_group=2,
              route_scale=2.5, expert_bias=bias, limit=1.5)
    r1, a = O.ffn_forward(x, gate, lambda j: experts[j], coding="grouped", **kw)
    r2, b = O.ffn_forward(x, gate, lambda j: experts[j], coding="loop", **kw)
    assert np.array_equal(r1.indices, r2.indices)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-13)
    for t in (0, 17, 39):
        row = O.token_output(x[t], r1.indices[t], r1.weights[t], lambda j: experts[j], 1.5)
        assert np.allclose(row, a[t], rtol=1e-12, atol=1e-13)


def test_single_expert_top1_is_dense_swiglu_mlp():
    # E = 1, K = 1, softmax: the layer is the dense gated MLP (DraftMLP)
    rng = np.random.default_rng(53)
    x = rng.standard_normal((7, 24)); gate = rng.standard_normal((1, 24))
    ex = _rand_experts(rng, 1, 24, 10)[0]
    r, out = O.ffn_forward(x, gate, lambda j: ex, n_experts=1, k=1)
    assert np.all(r.weights == 1.0) and np.all(r.indices == 0)
    xt = torch.from_numpy(x)
    gu = F.linear(xt, torch.from_numpy(ex.w_gate_up))
    ref = F.linear(F.silu(gu[:, :10]) * gu[:, 10:], torch.from_numpy(ex.w_down)).numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_clamp_definition_and_special_limits():
    g = np.array([10.0, -10.0, 3.0]); u = np.array([-9.0, 9.0, 2.0])
    got = O.swiglu(g, u, 7.0)
    want = [7.0 / (1 + math.exp(-7.0)) * -7.0, -10.0 / (1 + math.exp(10.0)) * 7.0,
            3.0 / (1 + math.exp(-3.0)) * 2.0]
    assert np.allclose(got, want, rtol=1e-15)
    # limit = inf is plain SwiGLU; limit = 0 zeroes the activation
    gg = torch.linspace(-20, 20, 101, dtype=torch.float64)
    uu = torch.linspace(15, -15, 101, dtype=torch.float64)
    assert np.allclose(O.swiglu(gg.numpy(), uu.numpy(), math.inf), (F.silu(gg) * uu).numpy(),
                       rtol=1e-14, atol=1e-300)
    assert np.all(O.swiglu(gg.numpy(), uu.numpy(), 0.0) == 0)


def test_swiglu_oai_closed_forms_and_identities():
    """gpt-oss's activation as read here: h = g sigma(1.702 g) (u + 1) on the
    clamped pre-activations (a reading, not the pages' definition: parity of
    this activation is unpinned by the pages)."""
    rng = np.random.default_rng(57)
    g = rng.uniform(-6.5, 6.5, 2000); u = rng.uniform(-9, 9, 2000)
    L = 7.0
    # zeros: the gate at 0, the linear factor at u = -1
    assert np.all(O.swiglu(np.zeros(5), rng.uniform(-5, 5, 5), L, "swiglu_oai") == 0)
    assert np.all(O.swiglu(rng.uniform(-5, 5, 5), np.full(5, -1.0), L, "swiglu_oai") == 0)
    # one value worked by hand: g = 1, u = 0 gives sigma(1.702) = 1 / (1 + 0.182319...) = 0.845796...
    assert abs(O.swiglu(np.array([1.0]), np.array([0.0]), L, "swiglu_oai")[0] - 0.8457957659) < 1e-9
    # odd part: sigma(z) + sigma(-z) = 1, so h(g, u) - h(-g, u) = g (u + 1) for |g| <= L
    uc = np.clip(u, -L, L)
    d = O.swiglu(g, u, L, "swiglu_oai") - O.swiglu(-g, u, L, "swiglu_oai")
    assert np.allclose(d, g * (uc + 1.0), rtol=1e-13, atol=1e-13)
    # the clamp: g above L acts as L, u outside [-L, L] as the bound
    assert np.array_equal(O.swiglu(g + 20.0, u, L, "swiglu_oai"), O.swiglu(np.full_like(g, L), u, L, "swiglu_oai"))
    assert np.array_equal(O.swiglu(g, np.where(u > 0, 30.0, -30.0), L, "swiglu_oai"),
                          O.swiglu(g, np.where(u > 0, L, -L), L, "swiglu_oai"))
    # tails without a clamp: g sigma(a g) -> g for large g, -> 0 for very negative g
    big = np.array([60.0, -60.0])
    h = O.swiglu(big, np.array([1.0, 1.0]), math.inf, "swiglu_oai")
    assert h[0] == 120.0 and abs(h[1]) < 1e-40
    # against torch's sigmoid (fp64), a library route to the logistic function
    gt, ut = torch.from_numpy(np.minimum(g, L)), torch.from_numpy(uc)
    ref = (gt * torch.sigmoid(1.702 * gt) * (ut + 1.0)).numpy()
    assert np.allclose(O.swiglu(g, u, L, "swiglu_oai"), ref, rtol=1e-14, atol=1e-14)


def test_zero_limit_leaves_only_shared_expert():
    rng = np.random.default_rng(54)
    x = rng.standard_normal((6, 16)); gate = rng.standard_normal((4, 16))
    experts = _rand_experts(rng, 4, 16, 8)
    shg, shd = 0.3 * rng.standard_normal((8, 16)), 0.3 * rng.standard_normal((16, 4))
    r, out = O.ffn_forward(x, gate, lambda j: experts[j], n_experts=4, k=2, limit=0.0,
                           sh_gate_up64=shg, sh_down64=shd)
    assert np.array_equal(out, O.shared_expert(x, shg, shd, 0.0, None))
    assert np.all(out == 0)          # the shared expert uses the same clamp


def test_zero_shared_gate_halves_the_shared_expert():
    rng = np.random.default_rng(55)
    x = rng.standard_normal((6, 16))
    shg, shd = 0.3 * rng.standard_normal((8, 16)), 0.3 * rng.standard_normal((16, 4))
    gated = O.shared_expert(x, shg, shd, math.inf, np.zeros(16))
    plain = O.shared_expert(x, shg, shd, math.inf, None)
    assert np.array_equal(gated, 0.5 * plain)


def test_mxfp4_expert_equals_dequantised_expert():
    # the MXFP4 expert is the bf16-style expert on the decoded weights
    rng = np.random.default_rng(56)
    h, i = 64, 32
    codes_gu = rng.integers(0, 256, size=(2 * i, h // 2)).astype(np.uint8)
    sc_gu = rng.integers(124, 128, size=(2 * i, h // 32)).astype(np.uint8)
    codes_d = rng.integers(0, 256, size=(h, i // 2)).astype(np.uint8)
    sc_d = rng.integers(124, 128, size=(h, i // 32)).astype(np.uint8)
    wgu = O.mxfp4_dequant(codes_gu, sc_gu); wd = O.mxfp4_dequant(codes_d, sc_d)
    # decode by explicit per-element loop (independent of the vectorised path)
    ref = np.zeros((2 * i, h))
    vals = _golden_e2m1()["values"]
    for n in range(2 * i):
        for k in range(h):
            b = int(codes_gu[n, k // 2]); c = (b >> 4) if (k & 1) else (b & 15)
            ref[n, k] = vals[c] * 2.0 ** (int(sc_gu[n, k // 32]) - 127)
    assert np.array_equal(wgu, ref)
    x = rng.standard_normal((3, h))
    y = O.expert_mlp(x, wgu, wd, 7.0)
    assert y.shape == (3, h) and np.all(np.isfinite(y))


def test_selection_margins():
    c = np.array([[0.9, 0.5, 0.4, 0.1]], dtype=F32)
    idx = O.select(c, 2)
    m = O.selection_margins(c, idx)
    assert abs(m[0] - (0.5 - 0.4)) < 1e-7


def test_selection_margins_group_worked_examples():
    # Two groups of four experts, keep one group, K = 2.  Dyadic values, so
    # every fp32 sum and difference below is exact.
    # (a) the group gap binds: group scores 0.875 + 0.25 = 1.125 and
    #     0.625 + 0.4375 = 1.0625 (gap 0.0625); inside the kept group the picks
    #     are experts 0, 1 and the best admissible value left is 0.125 (gap 0.125)
    a = np.array([[0.875, 0.25, 0.125, 0.0, 0.625, 0.4375, 0.25, 0.0625]], dtype=F32)
    ia = O.select(a, 2, n_group=2, topk_group=1)
    assert ia.tolist() == [[0, 1]]
    assert O.selection_margins(a, ia, 2, 1)[0] == 0.0625
    # (b) the within-group gap binds, and the dropped group's 0.5 (larger than
    #     every unpicked kept value) must not count: group scores 1.125 and
    #     0.875 (gap 0.25); picks 0, 1; best admissible left 0.1875 -> 0.0625
    b = np.array([[0.875, 0.25, 0.1875, 0.0, 0.5, 0.375, 0.25, 0.0625]], dtype=F32)
    ib = O.select(b, 2, n_group=2, topk_group=1)
    assert ib.tolist() == [[0, 1]]
    assert O.selection_margins(b, ib, 2, 1)[0] == 0.0625
    # (c) exact ties give a zero margin: equal group scores (1.125 both) ...
    c = np.array([[0.875, 0.25, 0.0, 0.0, 0.625, 0.5, 0.0, 0.0]], dtype=F32)
    assert O.selection_margins(c, O.select(c, 2, 2, 1), 2, 1)[0] == 0.0
    # ... and a kept-group value equal to the last pick
    d = np.array([[0.875, 0.25, 0.25, 0.0, 0.5, 0.375, 0.0, 0.0]], dtype=F32)
    assert O.selection_margins(d, O.select(d, 2, 2, 1), 2, 1)[0] == 0.0
    # (d) K covers every expert of the kept groups: only the group gap is left
    e = np.array([[0.875, 0.25, 0.625, 0.4375, 0.125, 0.0]], dtype=F32)
    ie = O.select(e, 4, n_group=3, topk_group=2)
    assert sorted(ie[0].tolist()) == [0, 1, 2, 3]
    assert O.selection_margins(e, ie, 3, 2)[0] == (0.625 + 0.4375) - (0.125 + 0.0)


def _margin_by_pairs(row, picked, n_group, topk_group):
    """Independent coding of the selection margin by enumeration: the smallest
    difference between a kept and a dropped group score (all pairs), and
    between a picked value and an admissible unpicked one (all pairs).  The
    kept groups are the topk_group-subset of largest score sum, ties broken
    by the lexicographically smallest group ids; group scores are re-derived
    by a scalar top-2 scan."""
    e = len(row)
    size = e // n_group
    gs = []
    for g in range(n_group):
        best, second = -math.inf, -math.inf
        for v in row[g * size:(g + 1) * size]:
            v = float(v)
            if v > best:
                best, second = v, best
            elif v > second:
                second = v
        gs.append(float(F32(F32(best) + F32(second))))
    m = math.inf
    admissible = set(range(e))
    if n_group > 1:
        subsets = list(itertools.combinations(range(n_group), topk_group))
        kept = max(subsets, key=lambda s: (sum(sorted((gs[g] for g in s))), [-g for g in s]))
        # the kept set must be the top groups individually as well
        dropped = [g for g in range(n_group) if g not in kept]
        for a in kept:
            for b in dropped:
                m = min(m, gs[a] - gs[b])
        admissible = {j for g in kept for j in range(g * size, (g + 1) * size)}
    picked = [int(p) for p in picked]
    for i in picked:
        for j in admissible:
            if j not in picked:
                m = min(m, float(row[i]) - float(row[j]))
    return m


def test_selection_margins_match_pairwise_enumeration():
    rng = np.random.default_rng(61)
    cases = [(8, 2, 1, 2), (8, 2, 1, 3), (12, 3, 2, 3), (12, 4, 2, 4), (12, 4, 3, 5),
             (12, 3, 1, 1), (9, 3, 2, 6), (12, 1, 1, 3)]
    for e, g, tg, k in cases:
        for trial in range(40):
            # coarse values make exact ties (within groups, between groups) common
            row = (rng.integers(0, 9, size=e) / 8.0).astype(F32) if trial % 2 else \
                rng.random(e).astype(F32)
            c = row[None, :]
            idx = O.select(c, k, g, tg)
            got = O.selection_margins(c, idx, g, tg)[0]
            want = _margin_by_pairs(row, idx[0], g, tg)
            assert got == want, (e, g, tg, k, row.tolist(), idx.tolist(), got, want)


def test_selection_margins_bound_the_stable_region():
    """Soundness: moving every selection value by less than margin/4 leaves the
    group-limited selection unchanged (group scores, sums of two values, move
    by less than margin/2).  Tightness: raising the best excluded candidate by
    slightly more than the margin changes it."""
    rng = np.random.default_rng(62)
    for e, g, tg, k in [(16, 4, 2, 3), (32, 8, 4, 8), (12, 3, 1, 2), (16, 1, 1, 4)]:
        for _ in range(60):
            row = rng.random(e).astype(np.float64)
            c = row.astype(F32)[None, :]
            idx = O.select(c, k, g, tg)
            m = O.selection_margins(c, idx, g, tg)[0]
            assert m > 0
            for _ in range(5):
                d = rng.uniform(-0.24 * m, 0.24 * m, size=e)
                c2 = (c.astype(np.float64) + d).astype(F32)
                if np.max(np.abs(c2.astype(np.float64) - c.astype(np.float64))) >= 0.25 * m:
                    continue     # fp32 rounding of the perturbed value
                # the selected set (the order of near-equal picks may change)
                assert np.array_equal(np.sort(O.select(c2, k, g, tg)), np.sort(idx))
            # tightness: push the candidate that defines the margin past it
            c3 = c.astype(np.float64).copy()[0]
            size = e // g
            gsc = O.group_scores(c[0], g).astype(np.float64) if g > 1 else None
            kept = [0]
            if g > 1:
                order = np.argsort(-gsc, kind="stable")
                kept = [int(x) for x in order[:tg]]
                group_gap = gsc[order[tg - 1]] - gsc[order[tg]] if tg < g else math.inf
            else:
                group_gap = math.inf
            adm = np.zeros(e, dtype=bool)
            for kg in kept:
                adm[kg * size:(kg + 1) * size] = True
            rest = adm.copy()
            rest[idx[0]] = False
            within_gap = c3[idx[0]].min() - c3[rest].max() if rest.any() else math.inf
            if within_gap <= group_gap:
                j = int(np.flatnonzero(rest)[np.argmax(c3[rest])])
                c3[j] += within_gap * 1.01 + 1e-6
            else:
                b = int(order[tg])                 # best dropped group: raise its top value
                top = b * size + int(np.argmax(c3[b * size:(b + 1) * size]))
                c3[top] += group_gap * 1.01 + 1e-6
            assert not np.array_equal(np.sort(O.select(c3.astype(F32)[None, :], k, g, tg)), np.sort(idx))


# ----------------------------------------------------------------------------
# Load-balancing state ([SF1073] commit notes on tokens_per_expert,
# moe/step_balance and update_expert_bias)
# ----------------------------------------------------------------------------
def test_masked_counts_match_bincount_of_kept_tokens():
    rng = np.random.default_rng(11)
    idx = rng.integers(0, 12, size=(50, 3)).astype(np.int32)
    mask = rng.random(50) < 0.6
    got = O.masked_expert_counts(idx, 12, mask)
    want = np.bincount(idx[mask].ravel(), minlength=12)
    assert np.array_equal(got, want)
    assert got.dtype == np.int64
    assert int(got.sum()) == 3 * int(mask.sum())
    # no mask keeps every token; an all-false mask keeps none
    assert np.array_equal(O.masked_expert_counts(idx, 12), O.expert_counts(idx, 12))
    assert not O.masked_expert_counts(idx, 12, np.zeros(50, bool)).any()


def test_step_balance_closed_forms():
    # uniform load -> 1; load collapsed onto K of E experts -> E / K
    assert O.step_balance(np.full(8, 5)) == 1.0
    E, K, T = 8, 2, 40
    collapsed = np.zeros(E, np.int64)
    collapsed[[3, 6]] = T
    assert O.step_balance(collapsed) == E / K
    # hand-worked: E * max / sum = 4 * 3 / 4
    assert O.step_balance(np.array([3, 1, 0, 0])) == 3.0
    # no kept slot: reported as uniform
    assert O.step_balance(np.zeros(6, np.int64)) == 1.0


def test_bias_sign_step_hand_worked():
    # counts [3, 1, 0, 0]: mean 1 -> s = [-1, 0, +1, +1], mean(s) = 1/4;
    # with rate 2^-10 every step is exact in fp32
    r = 2.0 ** -10
    b0 = np.array([0.5, -0.25, 0.0, 1.0], np.float32)
    got = O.update_expert_bias(b0, np.array([3, 1, 0, 0]), r)
    want = b0 + np.array([-1.25, -0.25, 0.75, 0.75], np.float32) * np.float32(r)
    assert np.array_equal(got, want)
    # zero-mean delta: the bias sum is unchanged (exact here)
    assert float(got.astype(np.float64).sum()) == float(b0.astype(np.float64).sum())


def test_bias_sign_step_invariants():
    rng = np.random.default_rng(5)
    b0 = rng.standard_normal(16).astype(np.float32) * np.float32(0.01)
    # rate 0 keeps a loaded bias fixed, bitwise (negative zeros included)
    b0[3] = np.float32(-0.0)
    counts = rng.integers(0, 100, 16)
    same = O.update_expert_bias(b0, counts, 0.0)
    assert same.tobytes() == b0.tobytes()
    # uniform load: every sign is 0, nothing moves
    assert np.array_equal(O.update_expert_bias(b0, np.full(16, 7), 0.01), b0)
    # overloaded experts go down, underloaded go up, ties with the mean stay
    counts = np.array([10, 0, 5, 5] * 4)
    new = O.update_expert_bias(np.zeros(16, np.float32), counts, 0.01)
    assert new[counts > 5].max() < new[counts == 5].min() and new[counts < 5].min() > new[counts == 5].max()
    # mean 5 exactly: the ties get -rate * mean(s) = 0
    assert (new[counts == 5] == 0).all()
    # the sign is decided on integers even when the mean is not an integer
    c = np.array([1, 2, 2])  # mean 5/3
    s = np.sign(c.mean() - c)
    new = O.update_expert_bias(np.zeros(3, np.float32), c, 1.0)
    want = (s - s.mean()).astype(np.float32)
    assert np.allclose(new, want, rtol=0, atol=1e-7)
