"""The seeded input generator: CPU and device code paths compute the same
integers, draws are reproducible, and the workload table has the sizes the
pages' workloads use."""

import numpy as np
import torch

from mixture_experts_ffn_04_amd import workloads as W


def test_u32_paths_agree():
    k1, k2 = W._keys(0, 5, 3)
    i = torch.arange(50000, dtype=torch.int64)
    ref = W._fmix32(W._fmix32(i + k1) ^ k2)          # the int64 (device) arithmetic
    assert torch.equal(ref, W.draw_u32(0, 5, 3, 50000))


def test_bf16_rounding_paths_agree_and_match_torch():
    f = W.draw_normal_f32(0, 1, 9, 20000, 1.0)
    b = f.view(torch.int32).to(torch.int64) & W.MASK32
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) & 0xFFFF
    assert torch.equal(r, W.f32_to_bf16_bits(f))
    assert torch.equal(f.to(torch.bfloat16).view(torch.int16),
                       W.draw_bf16(0, 1, 9, 20000, 1.0).view(torch.int16))


def test_draws_are_reproducible_and_distinct():
    a = W.draw_bf16(0, 5, 1, 4096, 0.02)
    assert torch.equal(a.view(torch.int16), W.draw_bf16(0, 5, 1, 4096, 0.02).view(torch.int16))
    assert not torch.equal(a.view(torch.int16), W.draw_bf16(0, 5, 2, 4096, 0.02).view(torch.int16))
    x = W.draw_normal_f32(0, 1, 0, 1 << 18, 1.0).numpy()
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01


def test_scales_and_codes_ranges():
    s = W.draw_e8m0(0, 14, 0, 10000, -3, 0).numpy()
    assert s.min() == 124 and s.max() == 127
    c = W.draw_bytes(0, 12, 0, 10000).numpy()
    assert c.min() == 0 and c.max() == 255


def test_workload_table():
    c2 = W.workload("qwen3_8b_moe_draft", T=72)
    assert (c2.H, c2.E, c2.I, c2.K) == (4096, 8, 1536, 1)
    c3 = W.workload("qwen3_5_moe_drafter", T=4096)
    assert (c3.E, c3.I, c3.K, c3.shared_I, c3.shared_gated) == (512, 512, 10, 2048, True)
    c4 = W.workload("deepseek_v4_style", T=72, score_fn="sqrtsoftplus")
    assert (c4.n_group, c4.topk_group, c4.route_scale, c4.swiglu_limit) == (8, 4, 2.5, 7.0)
    c5 = W.workload("gpt_oss_style_mxfp4", T=2048)
    e = W.gen_expert(c5.with_T(72), 3)
    assert e["codes_gate_up"].shape == (5760, 1440) and e["scales_down"].shape == (2880, 90)
