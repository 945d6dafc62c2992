"""GPU parity of the load-balancing state (moe_balance_count / moe_balance_update)
against the oracle: counts bit-exact, step balance and the fp32 bias step
bitwise, counts zeroed.  [SF1073] commit notes on tokens_per_expert, on
MoEBalancing's moe/step_balance and on update_expert_bias."""

import numpy as np
import pytest
import torch

from mixture_experts_ffn_04_amd import api
from mixture_experts_ffn_04_amd import workloads as W
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

# (name, T, K, E, skew, keep): draft serving sizes, the large-batch sizes,
# a crowded (collapsing) load, masks, one expert, the expert limit
CASES = [
    ("t72_e8_top1", 72, 1, 8, 1.0, 1.0),
    ("t72_e256_top8_masked", 72, 8, 256, 1.0, 0.7),
    ("t4096_e512_top10_masked", 4096, 10, 512, 1.0, 0.8),
    ("t8192_e8_top1", 8192, 1, 8, 1.0, 1.0),
    ("t3000_e1024_top16_crowded", 3000, 16, 1024, 6.0, 0.9),
    ("t1025_e1_top1", 1025, 1, 1, 1.0, 0.5),
    ("t300_e64_none_kept", 300, 4, 64, 1.0, 0.0),
]


def _np(t):
    return t.detach().cpu().numpy()


@pytest.mark.parametrize("name,T,K,E,skew,keep", CASES, ids=[c[0] for c in CASES])
def test_balance_matches_oracle(name, T, K, E, skew, keep):
    print(f"[balance] {name} T={T} K={K} E={E}", flush=True)
    idx, mask, bias = W.gen_balance_inputs(0, T, K, E, skew=skew, keep=keep)
    idx2, mask2, _ = W.gen_balance_inputs(0, T, K, E, skew=skew, keep=keep, sid=1)
    dev = "cuda"
    counts = torch.zeros(E, dtype=torch.int64, device=dev)
    # two forwards accumulate, the second without a mask
    api.balance_count(idx.to(dev), counts, mask.to(dev))
    api.balance_count(idx2.to(dev), counts, None)
    torch.cuda.synchronize()
    want = O.masked_expert_counts(_np(idx), E, _np(mask)) + O.masked_expert_counts(_np(idx2), E)
    got = _np(counts)
    assert np.array_equal(got, want), (got[:16], want[:16])

    b = bias.to(dev)
    rate = 1e-3
    sb = api.balance_update(counts, b, rate)
    torch.cuda.synchronize()
    assert _np(sb)[0] == np.float32(O.step_balance(want)), (_np(sb)[0], O.step_balance(want))
    want_b = O.update_expert_bias(_np(bias), want, rate)
    assert _np(b).tobytes() == want_b.tobytes(), np.max(np.abs(_np(b) - want_b))
    assert not _np(counts).any()
    print(f"[balance] {name}: step_balance {float(_np(sb)[0]):.4f}, kept slots {int(want.sum())}", flush=True)


def test_balance_rate_zero_keeps_bias_and_empty_count():
    E = 32
    idx, mask, bias = W.gen_balance_inputs(0, 100, 2, E)
    bias[5] = -0.0
    dev = "cuda"
    counts = torch.zeros(E, dtype=torch.int64, device=dev)
    api.balance_count(idx[:0].to(dev), counts, None)  # T = 0: nothing
    api.balance_count(idx.to(dev), counts, mask.to(dev))
    b = bias.to(dev)
    sb = api.balance_update(counts, b, 0.0)
    torch.cuda.synchronize()
    assert _np(b).tobytes() == _np(bias).tobytes()
    assert _np(sb)[0] == np.float32(O.step_balance(O.masked_expert_counts(_np(idx), E, _np(mask))))
    assert not _np(counts).any()
    # nothing counted: uniform, and no expert moves (the zero delta still
    # turns the planted -0.0 into +0.0, on both sides)
    sb = api.balance_update(counts, b, 0.5)
    torch.cuda.synchronize()
    want = O.update_expert_bias(_np(bias), np.zeros(E, np.int64), 0.5)
    assert _np(sb)[0] == 1.0 and _np(b).tobytes() == want.tobytes()
    assert np.array_equal(want, _np(bias))


def test_balance_collapsed_load_reports_e_over_k():
    E, K, T = 64, 4, 500
    idx = torch.tensor([[3, 17, 40, 63]] * T, dtype=torch.int32)
    dev = "cuda"
    counts = torch.zeros(E, dtype=torch.int64, device=dev)
    api.balance_count(idx.to(dev), counts)
    sb = api.balance_update(counts, None, 0.0)
    torch.cuda.synchronize()
    assert _np(sb)[0] == E / K
