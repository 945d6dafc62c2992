"""moe_ffn_forward_noalloc (the forward on the library's own scratch array)
against moe_ffn_forward (the forward on a caller's workspace), through the C
ABI: two calls in a row on one device, the second with a smaller batch, so
that the second runs on what the first left in the scratch array.  Both
entry points run the same kernels, so the results must agree bit for bit
(stronger than the 2e-2 x RMS bar of the bf16 outputs).  Oversized
configurations are refused on the host before anything is enqueued."""

import ctypes
import math

import pytest
import torch

from mixture_experts_ffn_04_amd import _lib, api
from mixture_experts_ffn_04_amd import workloads as W

pytestmark = pytest.mark.gpu

Wl = W.Workload

CASES = [
    Wl("noalloc_grouped_shared", T=72, H=512, E=64, I=160, K=6, score_fn="sigmoid", n_group=8,
       topk_group=4, route_scale=2.5, swiglu_limit=7.0, shared_I=128, shared_gated=True,
       expert_bias_std=0.05),
    Wl("noalloc_mxfp4", T=72, H=352, E=32, I=288, K=4, w_dtype="mxfp4", swiglu_limit=7.0,
       expert_linear_bias_std=0.02),
    Wl("noalloc_top1_direct", T=72, H=512, E=8, I=384, K=1),
]


def _pair(wl, T, lw):
    wl = wl.with_T(T)
    cfg = api.config_from_workload(wl)
    x = W.gen_x(wl, "cuda")
    r_ref = api.empty_routing(cfg)
    ref = api.ffn_forward(cfg, x, lw, routing=r_ref)
    r_na = api.empty_routing(cfg)
    out = torch.full_like(ref, float("nan"))
    api.ffn_forward_noalloc(cfg, x, lw, out=out, routing=r_na)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out.view(torch.int32),
                       ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref.view(torch.int32))
    assert torch.equal(r_na.indices, r_ref.indices)
    assert torch.equal(r_na.counts, r_ref.counts)
    assert torch.equal(r_na.scores.view(torch.int32), r_ref.scores.view(torch.int32))
    assert torch.equal(r_na.weights.view(torch.int32), r_ref.weights.view(torch.int32))


@pytest.mark.parametrize("wl", CASES, ids=[w.name for w in CASES])
def test_noalloc_matches_workspace_forward_twice(wl):
    print(f"[case] {wl.name}: T=72 then T=40 on the scratch array", flush=True)
    lw = api.layer_weights_from_workload(wl, "cuda")
    _pair(wl, 72, lw)
    _pair(wl, 40, lw)     # smaller batch on the first call's leftovers


def test_noalloc_refuses_oversized_config():
    wl = W.workload("deepseek_v4_style", T=4096)
    cfg = api.config_from_workload(wl)
    assert api.workspace_bytes(cfg) > _lib.NOALLOC_SCRATCH_BYTES
    dummy = ctypes.c_void_p(256)
    w = _lib.MoeWeights()
    st = _lib.lib().moe_ffn_forward_noalloc(ctypes.byref(cfg), dummy, ctypes.byref(w), dummy,
                                            None, None, None, None, None)
    assert st == _lib.MOE_ERR_WORKSPACE
    assert "no-allocation forward holds" in _lib.lib().moe_last_error().decode()
