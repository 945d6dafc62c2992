"""Pins of the oracle's backward of the layer (oracle/moe_oracle.py,
ffn_backward and its helpers).

The oracle writes every derivative out by hand.  These tests check it
against what does not share that arithmetic:
  - torch autograd through an independent torch coding of the forward (fp64,
    the oracle's selection held fixed),
  - central finite differences of that forward along random directions,
  - closed forms: a top-1 renormalised router has weight route_scale for
    every token, so no gradient reaches the gate; L = 0 makes every routed
    expert output its down bias only; the backward is linear in dout.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import moe_oracle as O

torch.set_default_dtype(torch.float64)


def make_case(seed, T=6, H=16, E=6, I=8, K=2, shared=True, gated=True, biases=False,
              router_bias=False, expert_bias=False):
    rng = np.random.default_rng(seed)
    c = dict(T=T, H=H, E=E, I=I, K=K)
    c["x"] = rng.standard_normal((T, H))
    c["gate"] = rng.standard_normal((E, H)) * 0.5
    c["wgu"] = rng.standard_normal((E, 2 * I, H)) * 0.4
    c["wd"] = rng.standard_normal((E, H, I)) * 0.4
    c["bgu"] = rng.standard_normal((E, 2 * I)) * 0.3 if biases else None
    c["bd"] = rng.standard_normal((E, H)) * 0.3 if biases else None
    c["sgu"] = rng.standard_normal((2 * 12, H)) * 0.4 if shared else None
    c["sd"] = rng.standard_normal((H, 12)) * 0.4 if shared else None
    c["sg"] = rng.standard_normal(H) * 0.3 if shared and gated else None
    c["rb"] = rng.standard_normal(E).astype(np.float32) * 0.2 if router_bias else None
    c["eb"] = rng.standard_normal(E).astype(np.float32) * 0.05 if expert_bias else None
    c["dout"] = rng.standard_normal((T, H))
    return c


def oracle_grads(c, **kw):
    def get(e):
        return O.ExpertWeights(c["wgu"][e], c["wd"][e],
                               None if c["bgu"] is None else c["bgu"][e],
                               None if c["bd"] is None else c["bd"][e])
    return O.ffn_backward(c["x"], c["gate"], get, c["dout"], n_experts=c["E"], k=c["K"],
                          expert_bias=c["eb"], router_bias=c["rb"], sh_gate_up64=c["sgu"],
                          sh_down64=c["sd"], sh_gate64=c["sg"], **kw)


def oracle_indices(c, **kw):
    sel = {k: v for k, v in kw.items() if k in ("score_fn", "n_group", "topk_group",
                                                  "norm_topk_prob", "route_scale")}
    return O.route(c["x"], c["gate"], k=c["K"], expert_bias=c["eb"], router_bias=c["rb"], **sel).indices


def torch_forward(c, idx, t, score_fn="softmax", norm_topk_prob=True, route_scale=1.0,
                  limit=math.inf, activation="swiglu", **_):
    """The layer in torch ops, selection `idx` fixed.  `t`: dict of leaf tensors."""
    logits = t["x"] @ t["gate"].T
    if "rb" in t:
        logits = logits + t["rb"]
    if score_fn == "softmax":
        s = torch.softmax(logits, dim=-1)
    elif score_fn == "sigmoid":
        s = torch.sigmoid(logits)
    else:
        s = torch.sqrt(F.softplus(logits, beta=1.0, threshold=60.0))
    ix = torch.as_tensor(idx, dtype=torch.long)
    picked = torch.gather(s, 1, ix)
    if norm_topk_prob:
        w = route_scale * picked / (picked.sum(dim=-1, keepdim=True) + 1e-20)
    else:
        w = route_scale * picked

    def mlp(xr, wgu, wd, bgu=None, bd=None):
        pre = xr @ wgu.T
        if bgu is not None:
            pre = pre + bgu
        g, u = pre.chunk(2, dim=-1)
        if not math.isinf(limit):
            g = torch.clamp(g, max=limit)
            u = torch.clamp(u, -limit, limit)
        if activation == "swiglu_oai":
            y = (g * torch.sigmoid(1.702 * g) * (u + 1.0)) @ wd.T
        else:
            y = (F.silu(g) * u) @ wd.T
        return y + bd if bd is not None else y

    rows = []
    for ti in range(c["T"]):
        acc = 0.0
        for kk in range(c["K"]):
            e = int(idx[ti, kk])
            y = mlp(t["x"][ti], t["wgu"][e], t["wd"][e], t["bgu"][e] if "bgu" in t else None,
                    t["bd"][e] if "bd" in t else None)
            acc = acc + w[ti, kk] * y
        rows.append(acc)
    out = torch.stack(rows)
    if "sgu" in t:
        sh = mlp(t["x"], t["sgu"], t["sd"])
        if "sg" in t:
            sh = torch.sigmoid(t["x"] @ t["sg"])[:, None] * sh
        out = out + sh
    return out


def leaves(c):
    t = {k: torch.tensor(c[k], requires_grad=True) for k in ("x", "gate", "wgu", "wd")}
    for k in ("bgu", "bd", "sgu", "sd", "sg"):
        if c[k] is not None:
            t[k] = torch.tensor(c[k], requires_grad=True)
    if c["rb"] is not None:
        t["rb"] = torch.tensor(c["rb"].astype(np.float64), requires_grad=True)
    return t


def torch_grads(c, idx, **kw):
    t = leaves(c)
    out = torch_forward(c, idx, t, **kw)
    (out * torch.tensor(c["dout"])).sum().backward()
    return {k: v.grad.numpy() for k, v in t.items()}


KW_CASES = [
    dict(score_fn="softmax"),
    dict(score_fn="sigmoid", route_scale=2.5),
    dict(score_fn="sqrtsoftplus", route_scale=1.5),
    dict(score_fn="softmax", norm_topk_prob=False),
    dict(score_fn="sigmoid", n_group=3, topk_group=2, route_scale=2.5),
    dict(score_fn="softmax", limit=0.7),
    dict(score_fn="softmax", limit=0.7, activation="swiglu_oai"),
    dict(score_fn="sigmoid", n_group=3, topk_group=2, route_scale=2.5, activation="swiglu_oai"),
]


@pytest.mark.parametrize("kw", KW_CASES, ids=[str(i) for i in range(len(KW_CASES))])
@pytest.mark.parametrize("variant", ["shared_gated", "biases_logitbias", "selbias_ungated"])
def test_backward_matches_autograd(kw, variant):
    opts = dict(shared_gated=dict(shared=True, gated=True),
                biases_logitbias=dict(shared=False, biases=True, router_bias=True),
                selbias_ungated=dict(shared=True, gated=False, expert_bias=True))[variant]
    c = make_case(3, **opts)
    g = oracle_grads(c, **kw)
    idx = oracle_indices(c, **kw)
    tg = torch_grads(c, idx, **kw)
    tol = dict(rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(g.dx, tg["x"], **tol)
    np.testing.assert_allclose(g.dgate, tg["gate"], **tol)
    for e in range(c["E"]):
        want_gu, want_d = tg["wgu"][e], tg["wd"][e]
        if e in g.dw_gate_up:
            np.testing.assert_allclose(g.dw_gate_up[e], want_gu, **tol)
            np.testing.assert_allclose(g.dw_down[e], want_d, **tol)
        else:  # an expert with no slot gets no gradient
            assert not want_gu.any() and not want_d.any()
    if c["bgu"] is not None:
        for e in g.db_gate_up:
            np.testing.assert_allclose(g.db_gate_up[e], tg["bgu"][e], **tol)
            np.testing.assert_allclose(g.db_down[e], tg["bd"][e], **tol)
    if c["rb"] is not None:
        np.testing.assert_allclose(g.drouter_bias, tg["rb"], **tol)
    if c["sgu"] is not None:
        np.testing.assert_allclose(g.dsh_gate_up, tg["sgu"], **tol)
        np.testing.assert_allclose(g.dsh_down, tg["sd"], **tol)
    if c["sg"] is not None:
        np.testing.assert_allclose(g.dsh_gate, tg["sg"], **tol)


@pytest.mark.parametrize("kw", [KW_CASES[1], KW_CASES[6]], ids=["sigmoid", "oai_clamp"])
def test_expert_grad_rows_match_autograd(kw):
    """expert_grad_rows (sampled weight-gradient entries from one expert's
    tokens) against autograd's full weight gradients, with biases and both
    activations; backward_routing_weights gives the weights it needs."""
    c = make_case(11, T=9, biases=True, router_bias=True)
    idx = oracle_indices(c, **kw)
    tg = torch_grads(c, idx, **kw)
    w = O.backward_routing_weights(c["x"], c["gate"], idx, router_bias=c["rb"],
                                   **{k: v for k, v in kw.items() if k in ("score_fn", "route_scale")})
    lim, act = kw.get("limit", math.inf), kw.get("activation", "swiglu")
    cols = np.array([0, 3, 7, 5])
    I = c["I"]
    seen = 0
    for e in range(c["E"]):
        tokens, slots = np.nonzero(idx == e)
        if tokens.size == 0:
            continue
        ew = O.ExpertWeights(c["wgu"][e], c["wd"][e], c["bgu"][e], c["bd"][e])
        gu, d = O.expert_grad_rows(c["x"], c["dout"], tokens, w[tokens, slots], ew, cols, limit=lim,
                                   activation=act)
        np.testing.assert_allclose(gu[0], tg["wgu"][e][cols], rtol=1e-9, atol=1e-11)
        np.testing.assert_allclose(gu[1], tg["wgu"][e][I + cols], rtol=1e-9, atol=1e-11)
        np.testing.assert_allclose(d, tg["wd"][e][:, cols], rtol=1e-9, atol=1e-11)
        seen += 1
    assert seen >= 3


def test_backward_matches_finite_differences():
    c = make_case(8, biases=True, router_bias=True)
    kw = dict(score_fn="sigmoid", route_scale=2.5)
    g = oracle_grads(c, **kw)
    idx = oracle_indices(c, **kw)
    rng = np.random.default_rng(1)
    dout = torch.tensor(c["dout"])

    def f(name, v, h):
        t = {k: x.detach().clone() for k, x in leaves(c).items()}
        t[name] = t[name] + h * torch.tensor(v)
        return float((torch_forward(c, idx, t, **kw) * dout).sum())

    h = 1e-5
    for name, grad in [("x", g.dx), ("gate", g.dgate), ("rb", g.drouter_bias),
                       ("sgu", g.dsh_gate_up), ("sg", g.dsh_gate)]:
        v = rng.standard_normal(grad.shape)
        fd = (f(name, v, h) - f(name, v, -h)) / (2 * h)
        an = float(np.sum(grad * v))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)
    e = int(idx[0, 0])
    v = np.zeros_like(c["wgu"])
    v[e] = rng.standard_normal(v[e].shape)
    fd = (f("wgu", v, h) - f("wgu", v, -h)) / (2 * h)
    an = float(np.sum(g.dw_gate_up[e] * v[e]))
    assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (fd, an)
    # the selection did not move under the perturbation (piecewise constant)
    xs = c["x"] + h * rng.standard_normal(c["x"].shape)
    assert np.array_equal(O.route(xs, c["gate"], k=c["K"], router_bias=c["rb"], **kw).indices, idx)


def test_top1_renormalised_router_gets_no_gradient():
    # K = 1 with renormalisation: w = route_scale * s / (s + eps) = route_scale
    c = make_case(4, K=1, shared=False, router_bias=True)
    g = oracle_grads(c, score_fn="softmax", route_scale=1.7)
    scale = np.abs(g.dx).max()
    assert np.abs(g.dgate).max() <= 1e-12 * scale
    assert np.abs(g.drouter_bias).max() <= 1e-12 * scale


def test_zero_limit_leaves_only_down_bias_and_shared():
    # L = 0: h = silu(min(g, 0)) * clip(u, 0, 0) = 0, so dW_down = 0 and the
    # routed experts pass no gradient to x through gate_up
    c = make_case(5, biases=True, shared=False)
    g = oracle_grads(c, limit=0.0)
    for e in g.dw_down:
        assert not g.dw_down[e].any()
        assert not g.dw_gate_up[e][c["I"]:].any()   # up rows: clip cuts every gradient
    # the router still sees y = b_down through the weights
    assert np.abs(g.dgate).max() > 0


def test_backward_is_linear_in_dout():
    c = make_case(6)
    g1 = oracle_grads(c)
    c2 = dict(c, dout=-2.5 * c["dout"])
    g2 = oracle_grads(c2)
    np.testing.assert_allclose(g2.dx, -2.5 * g1.dx, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g2.dgate, -2.5 * g1.dgate, rtol=1e-12, atol=1e-14)
    for e in g1.dw_gate_up:
        np.testing.assert_allclose(g2.dw_gate_up[e], -2.5 * g1.dw_gate_up[e], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("fn", ["softmax", "sigmoid", "sqrtsoftplus"])
def test_score_backward_matches_autograd(fn):
    rng = np.random.default_rng(2)
    l = rng.standard_normal(9) * 3
    ds = rng.standard_normal(9)
    lt = torch.tensor(l, requires_grad=True)
    s = {"softmax": lambda z: torch.softmax(z, 0), "sigmoid": torch.sigmoid,
         "sqrtsoftplus": lambda z: torch.sqrt(F.softplus(z, threshold=60.0))}[fn](lt)
    (s * torch.tensor(ds)).sum().backward()
    got = O.score_backward(l, s.detach().numpy(), ds, fn)
    np.testing.assert_allclose(got, lt.grad.numpy(), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("activation", ["swiglu", "swiglu_oai"])
def test_swiglu_backward_matches_autograd_with_clamp_on_both_sides(activation):
    rng = np.random.default_rng(9)
    g = rng.standard_normal(200) * 4
    u = rng.standard_normal(200) * 4
    dh = rng.standard_normal(200)
    for lim in (math.inf, 2.0):
        gt = torch.tensor(g, requires_grad=True)
        ut = torch.tensor(u, requires_grad=True)
        gc = gt if math.isinf(lim) else torch.clamp(gt, max=lim)
        uc = ut if math.isinf(lim) else torch.clamp(ut, -lim, lim)
        if activation == "swiglu":
            h = F.silu(gc) * uc
        else:
            h = gc * torch.sigmoid(1.702 * gc) * (uc + 1.0)
        (h * torch.tensor(dh)).sum().backward()
        dg, du = O.swiglu_backward(g, u, lim, dh, activation)
        np.testing.assert_allclose(dg, gt.grad.numpy(), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(du, ut.grad.numpy(), rtol=1e-12, atol=1e-14)
        if not math.isinf(lim):
            assert (dg[g > lim] == 0).all() and (du[np.abs(u) > lim] == 0).all()
