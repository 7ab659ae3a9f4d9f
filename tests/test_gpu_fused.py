"""GPU parity of leapq_append_fold (the window's last token and its fold in
one call) through the C ABI.

Free-running against the oracle, which appends and then folds, with the same
bar as tests/gpu_harness.py and bitwise fp32 equality.  At the headline
shape the fused path is also compared with the separate leapq_append +
leapq_fold path on every head of a layer.
"""
import dataclasses

import pytest
import torch

from quantized_recurrent_state_amd import leapq as lq
from quantized_recurrent_state_amd import workloads
from tests.gpu_harness import D, progress, run_layer

pytestmark = pytest.mark.gpu

WL = workloads.WORKLOADS


def _wl(base, **kw):
    return dataclasses.replace(WL[base], **kw)


def _finish(rep):
    progress(f"    summary: {rep.summary()}")
    rep.check()
    assert sum(rep.nonbit.values()) == 0, rep.nonbit


@pytest.mark.parametrize("name,wl,tokens", [
    ("tiny_f32", WL["tiny"], 64),
    ("tiny_bf16", _wl("tiny", in_dtype="bf16", seed=40), 48),
    ("W1", _wl("tiny", window=1, seed=41), 6),
    ("C8", _wl("tiny", n_comp=8, seed=42), 32),
    ("C0_nosmooth", _wl("tiny", n_comp=0, smoothing=False, seed=43), 32),
    ("W20_two_launches", _wl("tiny", window=20, seed=44), 40),
    ("ragged_heads", _wl("tiny", batch=3, heads=5, seed=45), 32),
    ("hard", _wl("tiny", init="hard", batch=1, heads=32, seed=46), 32),
])
def test_fused_against_oracle(name, wl, tokens):
    progress(f"  case {name}: {wl}")
    rep, L, _ = run_layer(wl, tokens=tokens, fused=True)
    assert L.n_records == tokens % wl.window
    _finish(rep)


def test_fused_full_size_b512_sampled():
    """The benchmark's launch shape: 64 sampled heads through 2 windows."""
    wl = WL["b512"]
    sample = list(range(11, 16384, 256))
    rep, _, _ = run_layer(wl, tokens=32, sample=sample, gen_device="cuda", check_every_token=False, fused=True)
    _finish(rep)


def test_fused_equals_separate_every_head_b512():
    """Two windows of one b512 layer: the fused path's outputs and boundary
    state equal the separate append + fold path's on all 16384 heads."""
    wl = WL["b512"]
    H = wl.batch * wl.heads
    cfg = lq.make_config(wl.batch, wl.heads, wl.window, wl.n_comp, wl.smoothing, wl.sigma_floor, wl.in_dtype)
    S0 = workloads.initial_state(wl, 0, device="cuda").reshape(H, D, D)
    La, Lb = lq.Layer(cfg, "cuda:0"), lq.Layer(cfg, "cuda:0")
    lq.leapq_init_state(La, S0)
    lq.leapq_init_state(Lb, S0)
    oa = torch.empty(H, D, device="cuda")
    ob = torch.empty_like(oa)
    mismatched_o = 0
    for t in range(2 * wl.window):
        q, k, v, a, b = workloads.token_inputs(wl, 0, t, device="cuda")
        q, k, v, a, b = q.reshape(H, D), k.reshape(H, D), v.reshape(H, D), a.reshape(H), b.reshape(H)
        lq.leapq_append(La, q, k, v, a, b, oa)
        if La.n_records == wl.window:
            lq.leapq_fold(La)
        if Lb.n_records == wl.window - 1:
            lq.leapq_append_fold(Lb, q, k, v, a, b, ob)
        else:
            lq.leapq_append(Lb, q, k, v, a, b, ob)
        mismatched_o += int((oa.view(torch.int32) != ob.view(torch.int32)).sum())
    torch.cuda.synchronize()
    assert La.n_records == Lb.n_records == 0
    progress(f"  outputs not bitwise equal: {mismatched_o}")
    assert mismatched_o == 0
    for name in ("codes_physical", "rho", "sigma", "comp_idx", "comp_vec"):
        x, y = getattr(La, name)(), getattr(Lb, name)()
        diff = int((x.view(torch.uint8) != y.view(torch.uint8)).sum()) if x.dtype == torch.int8 else \
            int((x.view(torch.int32) != y.view(torch.int32)).sum())
        progress(f"  {name}: {diff} differing elements")
        assert diff == 0, name
