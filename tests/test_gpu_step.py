"""GPU parity of leapq_step (a window phase per request) through the C ABI.

Requests start at different steps and some skip steps, so their window
phases differ: in one launch some heads append, some append and fold, and
some take no token.  Every active sampled head is checked against an oracle
head that appends and folds on its own request's schedule, with the bar of
tests/gpu_harness.py (bitwise on every fp32 value); the harness also checks
n_out and that output rows of idle requests are left untouched.
"""
import dataclasses

import numpy as np
import pytest
import torch

from quantized_recurrent_state_amd import leapq as lq
from quantized_recurrent_state_amd import workloads
from tests.gpu_harness import D, progress, run_staggered

pytestmark = pytest.mark.gpu

WL = workloads.WORKLOADS
GATE = dict(q_scale=128 ** -0.5, eps=1e-6)


def _wl(base, **kw):
    return dataclasses.replace(WL[base], **kw)


def _finish(rep):
    progress(f"    summary: {rep.summary()}")
    rep.check()
    assert sum(rep.nonbit.values()) == 0, rep.nonbit


def _skip_some(t, b):
    return (t + 3 * b) % 11 == 5


@pytest.mark.parametrize("name,wl,tokens,starts,kw", [
    ("f32", _wl("tiny", batch=4, heads=2, seed=110), 48, [0, 3, 7, 12], {}),
    ("bf16_W5", _wl("tiny", batch=4, heads=2, window=5, in_dtype="bf16", seed=111), 30, [0, 1, 2, 3], {}),
    ("gated_norm_bf16", _wl("tiny", batch=3, heads=3, in_dtype="bf16", seed=112), 40, [0, 5, 9],
     dict(gated=GATE, qk_norm=True)),
    ("gated_f32", _wl("tiny", batch=3, heads=2, seed=113), 36, [2, 0, 6], dict(gated=GATE)),
    ("kda", _wl("tiny_kda", batch=3, heads=2, seed=114), 40, [0, 4, 10], {}),
    ("bf16_records", _wl("tiny", batch=3, heads=2, in_dtype="bf16", seed=115), 40, [0, 6, 2], dict(rec_u="bf16")),
    ("fp8_records", _wl("tiny", batch=3, heads=2, in_dtype="bf16", seed=118), 40, [0, 6, 2], dict(rec_u="fp8")),
    ("rank1", _wl("tiny", batch=3, heads=2, seed=116, init="prefill"), 36, [0, 8, 3], dict(fit="rank1")),
    ("block", _wl("tiny", batch=3, heads=2, seed=117, init="prefill"), 36, [0, 8, 3], dict(fit="block")),
    ("C0_W1", _wl("tiny", batch=2, heads=2, window=1, n_comp=0, smoothing=False, seed=118), 8, [0, 2], {}),
])
def test_step_against_oracle(name, wl, tokens, starts, kw):
    progress(f"  case {name}: {wl}")
    rep, _, _, counts = run_staggered(wl, tokens, starts, skip=_skip_some, **kw)
    assert len(set(counts.tolist())) > 1 or wl.window == 1, counts  # the phases really differ
    _finish(rep)


def test_step_full_size_b512_sampled():
    """All 16,384 heads of a b512 layer with the requests' phases spread over
    the window (request b starts at step b % 16): every launch folds about a
    sixteenth of the requests.  64 sampled heads against the oracle."""
    wl = WL["b512"]
    starts = [b % 16 for b in range(wl.batch)]
    sample = list(range(9, 16384, 256))
    rep, _, _, _ = run_staggered(wl, 40, starts, sample=sample, gen_device="cuda", check_state=False)
    _finish(rep)


def test_step_in_phase_equals_append_calls():
    """With every request in phase, leapq_step equals leapq_append and
    leapq_append_fold bit for bit on every head of a b512 layer: outputs each
    token, and the boundary state and the records after a window, a fold and
    three more tokens."""
    wl = WL["b512"]
    H, dev = wl.batch * wl.heads, torch.device("cuda")
    cfg = lq.make_config(wl.batch, wl.heads, wl.window, wl.n_comp, wl.smoothing, wl.sigma_floor, wl.in_dtype)
    La, Ls = lq.Layer(cfg, dev), lq.Layer(cfg, dev)
    S0 = workloads.initial_state(wl, 0, device=dev).reshape(H, D, D)
    lq.leapq_init_state(La, S0)
    lq.leapq_init_state(Ls, S0)
    del S0
    oa = torch.empty(H, D, device=dev)
    os_ = torch.empty(H, D, device=dev)
    n_in = torch.zeros(wl.batch, dtype=torch.int32, device=dev)
    n_out = torch.empty_like(n_in)
    for t in range(wl.window + 3):
        q, k, v, a, b = (x.reshape(H, -1).squeeze(-1) for x in workloads.token_inputs(wl, 0, t, device=dev))
        if La.n_records == wl.window - 1:
            lq.leapq_append_fold(La, q, k, v, a, b, oa)
        else:
            lq.leapq_append(La, q, k, v, a, b, oa)
        lq.leapq_step(Ls, n_in, n_out, q, k, v, a, b, os_)
        assert torch.equal(oa.view(torch.int32), os_.view(torch.int32)), t
        assert torch.all(n_out == La.n_records), (t, La.n_records)
        n_in, n_out = n_out, n_in
    torch.cuda.synchronize()
    nb = int(La.layout.off_rec_gamma)  # codes, scales and compensators
    assert torch.equal(La.state[:nb], Ls.state[:nb])
    n = La.n_records
    for f in ("rec_gamma", "rec_k", "rec_u"):
        assert torch.equal(getattr(La, f)()[:, :n], getattr(Ls, f)()[:, :n]), f
    progress(f"  in phase: {wl.window + 3} tokens, outputs, boundary state and {n} records equal")


def test_step_out_of_range_phases_take_no_token():
    """Counts outside [0, W) (negative, W, far above) take no token: those
    requests' output rows and state bytes stay as they were, n_out echoes the
    count, and the other requests step normally; with n_out = NULL the step
    writes no counts."""
    wl = _wl("tiny", batch=4, heads=2, seed=119)
    H, dev = wl.batch * wl.heads, torch.device("cuda")
    cfg = lq.make_config(wl.batch, wl.heads, wl.window, wl.n_comp, wl.smoothing, wl.sigma_floor, wl.in_dtype)
    L, R = lq.Layer(cfg, dev), lq.Layer(cfg, dev)
    S0 = workloads.initial_state(wl, 0, device=dev).reshape(H, D, D)
    lq.leapq_init_state(L, S0)
    lq.leapq_init_state(R, S0)
    q, k, v, a, b = (x.reshape(H, -1).squeeze(-1).to(dev) for x in workloads.token_inputs(wl, 0, 0))
    before = L.state.clone()
    o = torch.full((H, D), float("nan"), device=dev)
    n_in = torch.tensor([-5, 0, 16, 1000], dtype=torch.int32, device=dev)
    n_out = torch.full((wl.batch,), 7, dtype=torch.int32, device=dev)
    lq.leapq_step(L, n_in, n_out, q, k, v, a, b, o)
    ref = torch.empty(H, D, device=dev)
    lq.leapq_append(R, q, k, v, a, b, ref)  # every request at n = 0
    torch.cuda.synchronize()
    assert n_out.tolist() == [-5, 1, 16, 1000]
    rows = torch.arange(H, device=dev) // wl.heads
    idle = rows != 1
    assert torch.all(torch.isnan(o[idle])) and torch.equal(o[~idle].view(torch.int32), ref[~idle].view(torch.int32))
    # an append leaves the boundary alone; request 1's record 0 equals the
    # append's, and the idle requests' record bytes are those from before
    for f in ("codes", "rho", "sigma", "comp_idx", "comp_vec"):
        assert torch.equal(getattr(L, f)(), getattr(R, f)()), f
    B0 = lq.Layer(cfg, dev)
    B0.state.copy_(before)
    hidle = idle.nonzero().flatten()
    for f in ("rec_gamma", "rec_k", "rec_u"):
        got, ref_f, old = getattr(L, f)(), getattr(R, f)(), getattr(B0, f)()
        assert torch.equal(got[~idle][:, 0], ref_f[~idle][:, 0]), f
        assert torch.equal(got[hidle].view(torch.int32), old[hidle].view(torch.int32)), f
    lq.leapq_step(L, torch.zeros(wl.batch, dtype=torch.int32, device=dev), None, q, k, v, a, b, o)
    torch.cuda.synchronize()
    assert not torch.any(torch.isnan(o))
