"""Host-side checks of the C ABI (no GPU needed, no kernel launched).

- the built library loads and exports every function include/moe_ffn.h
  declares;
- the ctypes structures have the exact layout the C compiler gives the
  header's structs (a small C program compiled with gcc prints it);
- moe_validate / moe_workspace_bytes refuse every invalid or unsupported
  configuration with the documented status;
- the entry points refuse bad pointers, aliasing and a short workspace before
  enqueueing anything.
"""

import ctypes
import math
import os
import re
import subprocess

import pytest

from mixture_experts_ffn_04_amd import _lib, api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_ffn.h")


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"MOE_API\s+[\w\s\*]*?\b(moe_\w+)\s*\(", src)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(_lib.EXPORTED)


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert set(declared_functions()) <= exported
    # nothing else is exported from the C ABI namespace
    assert {s for s in exported if s.startswith("moe_")} == set(declared_functions())


def test_abi_version(L):
    assert L.moe_abi_version() == _lib.ABI_VERSION


def test_struct_layout_matches_c(tmp_path):
    prog = tmp_path / "layout.c"
    prog.write_text(r'''
#include <stdio.h>
#include <stddef.h>
#include "moe_ffn.h"
#define F(s, m) printf(#s "." #m " %zu\n", offsetof(s, m));
int main(void) {
  printf("moe_config %zu\n", sizeof(moe_config));
  printf("moe_weights %zu\n", sizeof(moe_weights));
  F(moe_config, T) F(moe_config, H) F(moe_config, E) F(moe_config, I) F(moe_config, K)
  F(moe_config, act_dtype) F(moe_config, w_dtype) F(moe_config, score_fn)
  F(moe_config, n_group) F(moe_config, topk_group) F(moe_config, norm_topk_prob)
  F(moe_config, route_scale) F(moe_config, swiglu_limit) F(moe_config, shared_I)
  F(moe_config, shared_gated) F(moe_config, activation) F(moe_config, mx_gemm)
  F(moe_weights, gate_w) F(moe_weights, router_bias) F(moe_weights, expert_bias)
  F(moe_weights, w_gate_up) F(moe_weights, w_down) F(moe_weights, w_gate_up_scale)
  F(moe_weights, w_down_scale) F(moe_weights, b_gate_up) F(moe_weights, b_down)
  F(moe_weights, sh_gate_up) F(moe_weights, sh_down) F(moe_weights, sh_gate)
  printf("moe_grads %zu\n", sizeof(moe_grads));
  F(moe_grads, dx) F(moe_grads, dgate) F(moe_grads, drouter_bias) F(moe_grads, dw_gate_up)
  F(moe_grads, dw_down) F(moe_grads, db_gate_up) F(moe_grads, db_down) F(moe_grads, dsh_gate_up)
  F(moe_grads, dsh_down) F(moe_grads, dsh_gate)
  printf("enum %d %d %d %d %d %d %d %d %d %d %d %d %d\n", MOE_DTYPE_F32, MOE_DTYPE_BF16, MOE_DTYPE_MXFP4,
         MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID, MOE_SCORE_SQRTSOFTPLUS, MOE_OK, MOE_ERR_INVALID,
         MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP, MOE_ACT_SWIGLU, MOE_ACT_SWIGLU_OAI);
  return 0;
}
''')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-I", os.path.dirname(HEADER), str(prog), "-o", str(exe)],
                   check=True)
    got = dict(l.rsplit(" ", 1) for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                        check=True).stdout.splitlines()
               if not l.startswith("enum"))
    assert int(got["moe_config"]) == ctypes.sizeof(_lib.MoeConfig)
    assert int(got["moe_weights"]) == ctypes.sizeof(_lib.MoeWeights)
    for name, _ in _lib.MoeConfig._fields_:
        assert int(got[f"moe_config.{name}"]) == getattr(_lib.MoeConfig, name).offset, name
    for name, _ in _lib.MoeWeights._fields_:
        assert int(got[f"moe_weights.{name}"]) == getattr(_lib.MoeWeights, name).offset, name
    assert int(got["moe_grads"]) == ctypes.sizeof(_lib.MoeGrads)
    for name, _ in _lib.MoeGrads._fields_:
        assert int(got[f"moe_grads.{name}"]) == getattr(_lib.MoeGrads, name).offset, name
    enum_line = [l for l in subprocess.run([str(exe)], capture_output=True, text=True).stdout.splitlines()
                 if l.startswith("enum")][0]
    assert [int(v) for v in enum_line.split()[1:]] == [
        0, 1, 2, 0, 1, 2, _lib.MOE_OK, _lib.MOE_ERR_INVALID, _lib.MOE_ERR_UNSUPPORTED,
        _lib.MOE_ERR_WORKSPACE, _lib.MOE_ERR_HIP, _lib.MOE_ACT["swiglu"], _lib.MOE_ACT["swiglu_oai"]]


def cfg(**kw):
    base = dict(T=72, H=4096, E=8, I=1536, K=1)
    base.update({k: kw.pop(k) for k in list(kw) if k in base})
    return api.make_config(**base, **kw)


def status(L, c):
    return L.moe_validate(ctypes.byref(c))


def test_valid_configs(L):
    from mixture_experts_ffn_04_amd import workloads as W
    for fam, kw in W.FULL_CASES:
        c = api.config_from_workload(W.workload(fam, **kw))
        assert status(L, c) == 0, (fam, kw, L.moe_last_error())
        assert api.workspace_bytes(c) > 0
    assert status(L, cfg(T=0)) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), -1), (dict(H=0), -1), (dict(E=0), -1), (dict(I=-32), -1), (dict(K=0), -1),
    (dict(K=9), -1),
    (dict(E=8, n_group=0), -1), (dict(E=8, n_group=3), -1), (dict(E=8, n_group=2, topk_group=3), -1),
    (dict(E=8, n_group=2, topk_group=0), -1), (dict(E=8, n_group=8, topk_group=2), -1),
    (dict(E=16, K=5, n_group=4, topk_group=1), -1),
    (dict(route_scale=math.inf), -1), (dict(route_scale=math.nan), -1),
    (dict(swiglu_limit=math.nan), -1), (dict(swiglu_limit=-1.0), -1),
    (dict(shared_I=-32), -1),
    (dict(E=2048, K=2), -2), (dict(E=64, K=17), -2), (dict(E=256, n_group=128, topk_group=4, K=8), -2),
    (dict(H=4008), -2), (dict(I=1500), -2), (dict(shared_I=100), -2),
    (dict(act_dtype="f32", w_dtype="bf16"), -2), (dict(act_dtype="bf16", w_dtype="f32"), -2),
    (dict(act_dtype="f32", w_dtype="mxfp4"), -2),
])
def test_validate_refusals(L, kw, code):
    c = cfg(**kw)
    assert status(L, c) == code, (kw, L.moe_last_error())
    assert L.moe_last_error().decode()
    n = ctypes.c_size_t(0)
    assert L.moe_workspace_bytes(ctypes.byref(c), ctypes.byref(n)) == code


def test_bad_enum_values(L):
    for field, val in (("act_dtype", 7), ("w_dtype", 9), ("score_fn", 3), ("norm_topk_prob", 2),
                       ("shared_gated", 5), ("activation", 2), ("activation", -1), ("mx_gemm", 2),
                       ("mx_gemm", -1)):
        c = cfg()
        setattr(c, field, val)
        assert status(L, c) == -1, field


def test_workspace_grows_with_tokens():
    a = api.workspace_bytes(cfg(T=72))
    b = api.workspace_bytes(cfg(T=8192))
    assert 0 < a < b
    assert b >= 8192 * 4096 * 4          # at least the per-slot f32 expert outputs
    assert api.workspace_bytes(cfg(T=0)) >= 0


FAKE = 0x10000      # never dereferenced: every call below returns before enqueueing


def _fw(L, c, x=FAKE, out=FAKE + (1 << 30), ws=FAKE + (2 << 30), ws_bytes=1 << 40, **wkw):
    w = _lib.MoeWeights(gate_w=FAKE, w_gate_up=FAKE, w_down=FAKE)
    for k, v in wkw.items():
        setattr(w, k, v)
    return L.moe_ffn_forward(ctypes.byref(c), ctypes.c_void_p(x), ctypes.byref(w), ctypes.c_void_p(out),
                             None, None, None, None, ctypes.c_void_p(ws), ctypes.c_size_t(ws_bytes), None)


def test_forward_refuses_bad_arguments(L):
    c = cfg()
    assert _fw(L, c, x=0) == -1                     # NULL x
    assert _fw(L, c, out=0) == -1                   # NULL out
    assert _fw(L, c, x=FAKE + 8) == -1              # misaligned
    assert _fw(L, c, gate_w=0) == -1
    assert _fw(L, c, out=FAKE + 4096) == -1         # out overlaps x
    assert "overlaps" in L.moe_last_error().decode()
    assert _fw(L, c, ws=0) == -3
    assert _fw(L, c, ws_bytes=1000) == -3
    assert _fw(L, c, ws=FAKE + (2 << 30) + 64) == -3  # workspace alignment
    cs = cfg(shared_I=2048, shared_gated=True)
    assert _fw(L, cs, sh_gate_up=FAKE, sh_down=FAKE) == -1   # gated without sh_gate
    assert "sh_gate" in L.moe_last_error().decode()
    cm = cfg(H=2880, I=2880, E=32, K=4, w_dtype="mxfp4")
    assert _fw(L, cm) == -1                          # scales missing


def test_route_refuses_bad_arguments(L):
    c = cfg()
    P = ctypes.c_void_p
    args = [P(FAKE), P(FAKE), None, None, P(FAKE), P(FAKE), P(FAKE), None]
    assert L.moe_route(ctypes.byref(c), *args, P(FAKE), ctypes.c_size_t(10), None) == -3
    args[4] = None
    assert L.moe_route(ctypes.byref(c), *args, P(FAKE), ctypes.c_size_t(1 << 40), None) == -1
    assert L.moe_status_string(-3).decode() == "workspace missing or too small"


def test_balance_refuses_bad_arguments(L):
    P = ctypes.c_void_p
    f = ctypes.c_float
    # moe_balance_count(indices, mask, T, K, E, counts, stream): refused before any GPU work
    assert L.moe_balance_count(P(FAKE), None, -1, 2, 8, P(FAKE), None) == -1       # T < 0
    assert L.moe_balance_count(P(FAKE), None, 10, 0, 8, P(FAKE), None) == -1       # K = 0
    assert L.moe_balance_count(P(FAKE), None, 10, 2, 0, P(FAKE), None) == -1       # E = 0
    assert L.moe_balance_count(P(FAKE), None, 10, 2, 2048, P(FAKE), None) == -2    # E above the limit
    assert L.moe_balance_count(None, None, 10, 2, 8, P(FAKE), None) == -1          # NULL indices
    assert L.moe_balance_count(P(FAKE), None, 10, 2, 8, None, None) == -1          # NULL counts
    assert L.moe_balance_count(P(FAKE), None, 10, 2, 8, P(FAKE + 4), None) == -1   # counts misaligned
    assert "8-byte" in L.moe_last_error().decode()
    assert L.moe_balance_count(None, None, 0, 2, 8, P(FAKE), None) == 0            # T = 0: no work
    # moe_balance_update(counts, bias, E, rate, balance, stream)
    assert L.moe_balance_update(P(FAKE), P(FAKE), 0, f(0.1), None, None) == -1     # E = 0
    assert L.moe_balance_update(P(FAKE), P(FAKE), 4096, f(0.1), None, None) == -2  # E above the limit
    assert L.moe_balance_update(None, P(FAKE), 8, f(0.1), None, None) == -1        # NULL counts
    assert L.moe_balance_update(P(FAKE), None, 8, f(0.1), None, None) == -1        # rate without a bias
    assert "expert_bias" in L.moe_last_error().decode()
    assert L.moe_balance_update(P(FAKE), P(FAKE), 8, f(math.nan), None, None) == -1
    assert L.moe_balance_update(P(FAKE), P(FAKE + 2), 8, f(0.1), None, None) == -1  # bias misaligned


def test_backward_refuses_bad_arguments(L):
    P = ctypes.c_void_p
    c = cfg()
    w = _lib.MoeWeights(gate_w=FAKE, w_gate_up=FAKE, w_down=FAKE)
    g = _lib.MoeGrads(dx=FAKE, dgate=FAKE, dw_gate_up=FAKE, dw_down=FAKE)
    ws_bytes = ctypes.c_size_t()
    assert L.moe_backward_workspace_bytes(ctypes.byref(c), ctypes.byref(ws_bytes)) == 0 and ws_bytes.value > 0

    def bw(cc=c, ww=w, gg=g, ws=FAKE + (2 << 30), nbytes=1 << 40):
        return L.moe_ffn_backward(ctypes.byref(cc), P(FAKE), ctypes.byref(ww), P(FAKE), P(FAKE), P(FAKE),
                                  ctypes.byref(gg) if gg is not None else None, P(ws), ctypes.c_size_t(nbytes), None)
    assert bw(gg=None) == -1
    assert bw(gg=_lib.MoeGrads(dx=FAKE, dgate=FAKE, dw_gate_up=FAKE)) == -1          # dw_down missing
    assert bw(ww=_lib.MoeWeights(gate_w=FAKE, w_gate_up=FAKE, w_down=FAKE, router_bias=FAKE)) == -1
    assert "drouter_bias" in L.moe_last_error().decode()
    assert bw(nbytes=100) == -3
    assert bw(ws=FAKE + (2 << 30) + 64) == -3
    assert bw(cc=cfg(H=2880, I=2880, E=32, K=4, w_dtype="mxfp4")) == -2              # MXFP4 experts
    cs = cfg(shared_I=2048, shared_gated=True)
    assert bw(cc=cs, ww=_lib.MoeWeights(gate_w=FAKE, w_gate_up=FAKE, w_down=FAKE, sh_gate_up=FAKE,
                                        sh_down=FAKE, sh_gate=FAKE)) == -1            # dsh_* missing


def test_profile_stage_refusals(L):
    """moe_profile_stage refuses a stage past the last and missing events,
    and disarms with a negative stage; none of this touches the GPU."""
    ev = (ctypes.c_void_p * 2)(FAKE, FAKE)
    assert L.moe_profile_stage(len(_lib.STAGES), ev, ev, 2) == _lib.MOE_ERR_INVALID
    assert L.moe_profile_stage(0, None, None, 2) == _lib.MOE_ERR_INVALID
    assert L.moe_profile_stage(0, ev, ev, 0) == _lib.MOE_ERR_INVALID
    assert L.moe_profile_stage(-1, None, None, 0) == _lib.MOE_OK
