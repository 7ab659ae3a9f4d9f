"""GPU parity of the per-channel decay (KDA) path through the C ABI.

With LEAPQ_DECAY_CHANNEL the decay alpha is a 128-vector per head and token
("LeapQuant" App. A: D_t = Diag(alpha_t)), records carry cumulative decay
vectors, and every read and the fold's rebuild scale per key row.  The runs
are free-running against the oracle's KDA functions with the bar of
tests/gpu_harness.py, bitwise on every fp32 value; the dense fp32-state KDA
baseline is checked against the oracle's dense step.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from quantized_recurrent_state_amd import leapq as lq
from quantized_recurrent_state_amd import workloads
from tests.gpu_harness import D, progress, rel, run_layer

pytestmark = pytest.mark.gpu

WL = workloads.WORKLOADS


def _wl(base, **kw):
    return dataclasses.replace(WL[base], **kw)


def _finish(rep):
    progress(f"    summary: {rep.summary()}")
    rep.check()
    assert sum(rep.nonbit.values()) == 0, rep.nonbit


@pytest.mark.parametrize("name,wl,tokens,fused", [
    ("f32", WL["tiny_kda"], 64, False),
    ("f32_fused", _wl("tiny_kda", seed=60), 48, True),
    ("bf16_fused", _wl("tiny_kda", in_dtype="bf16", seed=61), 48, True),
    ("bf16", _wl("tiny_kda", in_dtype="bf16", seed=62), 37, False),
    ("W1", _wl("tiny_kda", window=1, seed=63), 6, False),
    ("W20_two_launches", _wl("tiny_kda", window=20, seed=64), 40, True),
    ("W64", _wl("tiny_kda", window=64, seed=65, init="prefill"), 64, False),
    ("C0_nosmooth", _wl("tiny_kda", n_comp=0, smoothing=False, seed=66), 32, True),
    ("C8", _wl("tiny_kda", n_comp=8, seed=67), 32, False),
    ("ragged_heads", _wl("tiny_kda", batch=3, heads=5, seed=68), 32, True),
])
def test_kda_against_oracle(name, wl, tokens, fused):
    progress(f"  case {name}: {wl}")
    rep, L, _ = run_layer(wl, tokens=tokens, fused=fused)
    assert L.n_records == tokens % wl.window
    _finish(rep)


def test_kda_dequant_views():
    wl = _wl("tiny_kda", seed=69, init="prefill")
    H = wl.batch * wl.heads
    rep, L, refs = run_layer(wl, tokens=21)  # one fold, then 5 records
    assert L.n_records == 5
    out = torch.empty(H, D, D, device="cuda")
    for what in (0, 1, 2):
        lq.leapq_dequant(L, what, out)
        got = out.cpu().numpy()
        for h in range(H):
            rep.fp(f"dequant{what}", got[h], refs[h].dequant(what))
    _finish(rep)


def test_kda_dense_baseline():
    """Dense fp32-state KDA decode against the oracle's dense step, 8 tokens."""
    wl = _wl("tiny_kda", batch=2, heads=16, init="prefill", seed=70)
    H = wl.batch * wl.heads
    cfg = lq.make_config(wl.batch, wl.heads, decay="channel")
    S0 = workloads.initial_state(wl, 0).reshape(H, D, D)
    S = S0.cuda().contiguous()
    ref = [S0[h].numpy().copy() for h in range(H)]
    o = torch.empty(H, D, device="cuda")
    eo = 0.0
    for t in range(8):
        q, k, v, a, b = workloads.token_inputs(wl, 0, t)
        q, k, v = (x.reshape(H, D) for x in (q, k, v))
        a, b = a.reshape(H, D), b.reshape(H)
        lq.leapq_gdn_decode(cfg, S, q.cuda(), k.cuda(), v.cuda(), a.cuda(), b.cuda(), o)
        og = o.cpu().numpy()
        for h in range(H):
            _, oref = oracle.kda_step_f32(ref[h], q[h].numpy(), k[h].numpy(), v[h].numpy(), a[h].numpy(),
                                          b[h].item())
            eo = max(eo, rel(og[h], oref))
    Sg = S.cpu().numpy()
    es = max(rel(Sg[h], ref[h]) for h in range(H))
    progress(f"    kda dense: output rel {eo:.2e}, state rel {es:.2e}")
    assert eo < 1e-5 and es < 1e-5


def test_kda_full_size_b512_every_head():
    """A whole b512 KDA layer, every head in the oracle: one window in the
    benchmark's schedule, all outputs and, after the fold, the whole
    boundary state bit for bit."""
    wl = WL["b512_kda"]
    rep, _, _ = run_layer(wl, tokens=wl.window, sample=None, gen_device="cuda", check_every_token=False,
                          fused=True)
    _finish(rep)


def test_kda_full_size_b512_sampled():
    """The KDA benchmark's launch shape (512 x 32 heads, bf16 inputs): 64
    sampled heads through 2 windows, the fused last token included."""
    wl = WL["b512_kda"]
    sample = list(range(9, 16384, 256))
    rep, _, _ = run_layer(wl, tokens=32, sample=sample, gen_device="cuda", check_every_token=False, fused=True)
    _finish(rep)


def test_kda_long_horizon_layer0():
    """4095 tokens (255 folds) of the per-channel decay study's first layer,
    with 4 oracle heads run free beside the GPU through the per-token hook of
    quantized_recurrent_state_amd.quality: bitwise equal outputs at every
    token.  The error against the fp32-state KDA recurrence is printed for the
    record and must be finite."""
    from quantized_recurrent_state_amd import quality
    wl = WL["long_kda"]
    heads_idx = (0, 7, 100, 255)
    S0 = workloads.initial_state(wl, 0, device="cuda").reshape(-1, D, D)[list(heads_idx)].cpu().numpy()
    heads = [oracle.Head(wl.n_comp, wl.window, wl.smoothing, wl.sigma_floor, decay="channel").init(S0[j])
             for j in range(len(heads_idx))]
    stat = {"non_bitwise": 0, "values": 0, "folds": 0}
    idx = torch.tensor(heads_idx, device="cuda")

    def on_token(layer, t, inputs, o, folded):
        q, k, v, a, b = (x.index_select(0, idx).float().cpu().numpy() for x in inputs)
        og = o.index_select(0, idx).cpu().numpy()
        for j, st in enumerate(heads):
            o_ref, _ = st.append(q[j], k[j], v[j], a[j], float(b[j]))
            stat["non_bitwise"] += int(np.sum(og[j].view(np.uint32) != np.asarray(o_ref, np.float32).view(np.uint32)))
            stat["values"] += D
            if folded:
                st.fold()
        stat["folds"] += int(folded)
        if (t + 1) % 1024 == 0:
            progress(f"  token {t + 1}: oracle agreement so far {stat}")

    res = quality.run("long_kda", layers=1, on_token=on_token, log=progress)
    progress(f"  quality: {res}")
    assert stat["folds"] == 255 and stat["non_bitwise"] == 0
    assert res["finite"]
