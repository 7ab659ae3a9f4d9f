"""GPU parity of libleapq against the CPU oracle (through the C ABI).

Free-running from the same seeded inputs; the bar is in tests/gpu_harness.py
(compensator indices exact, codes bit-exact up to the .5-boundary exemption,
fp32 within 1e-4 relative).  The harness also counts non-bitwise fp32 values;
the kernels follow the oracle's operation order, so these tests additionally
require them to be zero.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from quantized_recurrent_state_amd import leapq as lq
from quantized_recurrent_state_amd import workloads
from tests.gpu_harness import D, Report, progress, rel, run_layer

pytestmark = pytest.mark.gpu

WL = workloads.WORKLOADS


def _wl(base, **kw):
    return dataclasses.replace(WL[base], **kw)


def _finish(rep, bitwise=True):
    progress(f"    summary: {rep.summary()}")
    rep.check()
    if bitwise:
        assert sum(rep.nonbit.values()) == 0, rep.nonbit


def test_device_is_gfx950():
    assert torch.cuda.is_available()
    name = torch.cuda.get_device_properties(0).gcnArchName
    progress(f"device: {torch.cuda.get_device_name(0)} {name}")
    assert name.startswith("gfx950")
    assert lq.leapq_version() == 100


def test_init_tiny():
    rep, _, _ = run_layer(WL["tiny"], tokens=0)
    _finish(rep)


def test_window_tiny_f32():
    """1 request x 4 heads, 64 tokens = 4 folds, every token compared."""
    rep, _, _ = run_layer(WL["tiny"])
    _finish(rep)


def test_window_tiny_bf16_inputs():
    rep, _, _ = run_layer(_wl("tiny", in_dtype="bf16", seed=20), tokens=48)
    _finish(rep)


def test_window_b32_sampled():
    """Batch 32 x 32 heads (1024 heads, several tiles and XCD rounds) from the
    prefilled, outlier-injected initial state: 64 sampled heads through all
    256 tokens (16 folds)."""
    sample = list(range(0, 1024, 16))
    rep, _, _ = run_layer(WL["b32"], sample=sample, gen_device="cuda", check_every_token=False)
    _finish(rep)


@pytest.mark.parametrize("name,kw,tokens,fold_at", [
    ("W1", dict(window=1), 6, None),
    ("C0_nosmooth", dict(n_comp=0, smoothing=False), 32, None),
    ("C8", dict(n_comp=8), 32, None),
    ("C1_nosmooth", dict(n_comp=1, smoothing=False), 20, None),
    ("W20", dict(window=20), 40, None),
    ("W64", dict(window=64), 70, None),
    ("partial_window", dict(), 23, {5, 6, 17}),
    ("ragged_heads", dict(batch=3, heads=5), 18, None),
    ("one_head", dict(batch=1, heads=1, init="prefill"), 17, None),
    ("hard", dict(init="hard", batch=1, heads=32, seed=4), 33, None),
])
def test_edge_cases(name, kw, tokens, fold_at):
    wl = _wl("tiny", **{"seed": 30, **kw})
    progress(f"  case {name}: {wl}")
    rep, _, _ = run_layer(wl, tokens=tokens, fold_at=fold_at)
    _finish(rep)


def test_zero_state_and_empty_fold():
    wl = _wl("tiny", seed=31)
    H = wl.batch * wl.heads
    cfg = lq.make_config(wl.batch, wl.heads)
    L = lq.Layer(cfg)
    lq.leapq_init_state(L, torch.zeros(H, D, D, device="cuda"))
    lq.leapq_fold(L)  # fold with no records: requantizes the boundary
    torch.cuda.synchronize()
    ref = oracle.Head().init(np.zeros((D, D), np.float32)).fold()
    for h in range(H):
        assert np.array_equal(L.codes()[h].cpu().numpy(), ref.Q)
        assert np.array_equal(L.rho()[h].cpu().numpy(), ref.rho)
        assert np.array_equal(L.sigma()[h].cpu().numpy(), ref.sigma)
        assert list(L.comp_idx()[h].cpu().numpy()) == [-1] * 4
    assert L.n_records == 0


def test_code_rounds_exact_product_once():
    """The hand-derived fixture row (an entry a sliver above a .5 tie after
    scaling) quantized on the GPU: code 65 as the oracle and the fixture say,
    where rounding the fp32 product first would give 64.  Placed in a
    different row and head each time, without smoothing and compensators."""
    import json
    import os
    case = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "arith_fixtures.json")))[
        "round_exact_product_once"]
    H = 4
    cfg = lq.make_config(1, H, n_comp=0, smoothing=False)
    L = lq.Layer(cfg)
    S0 = np.zeros((H, D, D), np.float32)
    rows = [40, 3, 77, 127]
    for h, r in enumerate(rows):
        for i, x in case["row"].items():
            S0[h, r, (int(i) + 9 * h) % D] = np.float32(x)
    lq.leapq_init_state(L, torch.from_numpy(S0).cuda())
    torch.cuda.synchronize()
    Q = L.codes().cpu().numpy()
    rho = L.rho().cpu().numpy()
    for h, r in enumerate(rows):
        ref = oracle.Head(C=0, smoothing=False).init(S0[h])
        assert np.array_equal(Q[h], ref.Q) and np.array_equal(rho[h], ref.rho)
        for i, c in case["expected_codes"].items():
            assert int(Q[h, r, (int(i) + 9 * h) % D]) == c
        assert rho[h, r] == np.float32(case["expected_rho"])


def test_symmetric_states_tie_rows_and_columns():
    """Symmetric states: row i and column i hold the same entries in the same
    canonical order, so every row energy ties its column's.  The greedy pick
    takes the row (rows first), and the next pick meets the stale energies of
    the columns at their maximum, which must be rescored before picking again.
    Codes, scales, indices and lines bitwise against the oracle."""
    H = 8
    rng = np.random.default_rng(41)
    S0 = np.empty((H, D, D), np.float32)
    for h in range(H):
        A = rng.standard_normal((D, D)).astype(np.float32) * np.float32(0.02)
        for r in rng.choice(D, size=1 + h % 3, replace=False):
            A[r, :] *= np.float32(30.0 + 10.0 * h)
        S0[h] = np.triu(A) + np.triu(A, 1).T  # exactly symmetric
    cfg = lq.make_config(1, H)
    L = lq.Layer(cfg)
    lq.leapq_init_state(L, torch.from_numpy(S0).cuda())
    torch.cuda.synchronize()
    Q, rho, sig = L.codes().cpu().numpy(), L.rho().cpu().numpy(), L.sigma().cpu().numpy()
    idx, vec = L.comp_idx().cpu().numpy(), L.comp_vec().cpu().numpy()
    for h in range(H):
        ref = oracle.Head().init(S0[h])
        assert list(idx[h]) == list(ref.idx), (h, list(idx[h]), list(ref.idx))
        assert np.array_equal(vec[h].view(np.uint32), ref.vec.view(np.uint32))
        assert np.array_equal(Q[h], ref.Q) and np.array_equal(rho[h], ref.rho) and np.array_equal(sig[h], ref.sigma)


def test_dequant_all_views():
    wl = _wl("tiny", seed=32, init="prefill")
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


@pytest.mark.parametrize("state_dtype,in_dtype", [(torch.float32, "f32"), (torch.float32, "bf16"),
                                                  (torch.bfloat16, "f32"), (torch.bfloat16, "bf16")])
def test_gdn_baselines(state_dtype, in_dtype):
    """Dense per-token decode against the oracle's dense step, 8 tokens."""
    wl = _wl("tiny", batch=2, heads=16, init="prefill", in_dtype=in_dtype, seed=33)
    H = wl.batch * wl.heads
    cfg = lq.make_config(wl.batch, wl.heads, in_dtype=in_dtype)
    S0 = workloads.initial_state(wl, 0).reshape(H, D, D)
    S = S0.to(state_dtype).cuda().contiguous()
    if state_dtype == torch.bfloat16:
        ref = [S0[h].to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy() for h in range(H)]
    else:
        ref = [S0[h].numpy().copy() for h in range(H)]
    o = torch.empty(H, D, device="cuda")
    eo = es = 0.0
    for t in range(8):
        q, k, v, a, b = workloads.token_inputs(wl, 0, t)
        q, k, v = (x.reshape(H, D) for x in (q, k, v))
        a, b = a.reshape(H), b.reshape(H)
        lq.leapq_gdn_decode(cfg, S, q.cuda(), k.cuda(), v.cuda(), a.cuda(), b.cuda(), o)
        og = o.cpu().numpy()
        qw, kw_, vw = (workloads.widen(x).numpy() for x in (q, k, v))
        for h in range(H):
            step = oracle.gdn_step_bf16 if state_dtype == torch.bfloat16 else oracle.gdn_step_f32
            _, oref = step(ref[h], qw[h], kw_[h], vw[h], a[h].item(), b[h].item())
            eo = max(eo, rel(og[h], oref))
    Sg = S.float().cpu().numpy()
    for h in range(H):
        Sr = ref[h]
        if state_dtype == torch.bfloat16:
            Sr = oracle.bf16_bits_to_f32(Sr).reshape(D, D)
        es = max(es, rel(Sg[h], Sr))
    progress(f"    gdn {state_dtype} {in_dtype}: output rel {eo:.2e}, state rel {es:.2e}")
    if state_dtype == torch.float32:
        assert eo < 1e-5 and es < 1e-5
    else:
        # The baseline sums S^T k and S^T q in another order than the
        # oracle's sequential chain, so an fp32 value may land on the other
        # side of a bf16 rounding boundary: a stored entry then differs by
        # one bf16 unit (2^-8 relative), and later tokens carry it on.  The
        # bar allows a few such units.
        assert eo < 1e-2 and es < 1e-2


def test_full_size_b512_layer_sampled():
    """One layer at the headline batch (512 x 32 heads, bf16 inputs), the
    launch shape the benchmark times; 64 sampled heads through 2 windows."""
    wl = WL["b512"]
    sample = list(range(7, 16384, 256))
    rep, _, _ = run_layer(wl, tokens=32, sample=sample, gen_device="cuda", check_every_token=False)
    _finish(rep)


def test_full_size_b512_layer_every_head():
    """One whole b512 layer (16,384 heads, bf16 inputs) through one window in
    the benchmark's schedule (15 appends, then the last append and the fold
    in one launch), every head in the oracle: all 33.5M outputs and, after
    the fold, all 268M codes with their scales, compensator indices and
    lines, compared bit for bit."""
    wl = WL["b512"]
    rep, _, _ = run_layer(wl, tokens=wl.window, sample=None, gen_device="cuda", check_every_token=False,
                          fused=True)
    _finish(rep)


def test_full_size_b128_layer_sampled():
    wl = WL["b128"]
    sample = list(range(3, 4096, 64))
    rep, _, _ = run_layer(wl, layer=5, tokens=32, sample=sample, gen_device="cuda", check_every_token=False)
    _finish(rep)
