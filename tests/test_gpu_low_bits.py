"""GPU parity of the 6- and 4-bit residual states (state_bits = 6 or 4)
through the C ABI.

The residual keeps symmetric codes of -31 .. 31 or -7 .. 7 (scale absmax / 31
or / 7), packed in the layout of include/leapq.h (nibbles, plus 2-bit planes
at 6 bits); everything else is the int8 path.  Runs are free-running against
the oracle's bits=6 / bits=4 heads with the bar of tests/gpu_harness.py,
bitwise on every fp32 value; the binding unpacks the stored codes for the
comparison.  Edge cases from tests/test_gpu_edge.py (exact ties, tiny and
subnormal rows, fma-sensitive folds) run at both widths too.
"""
import dataclasses

import numpy as np
import pytest
import torch

from quantized_recurrent_state_amd import leapq as lq
from quantized_recurrent_state_amd import workloads
from tests.gpu_harness import D, Twin, progress, run_layer
from tests import test_gpu_edge as edge

pytestmark = pytest.mark.gpu

WL = workloads.WORKLOADS


def _wl(base, **kw):
    return dataclasses.replace(WL[base], **kw)


def _finish(rep):
    progress(f"    summary: {rep.summary()}")
    rep.check()
    assert sum(rep.nonbit.values()) == 0, rep.nonbit


@pytest.mark.parametrize("bits", [6, 4])
@pytest.mark.parametrize("name,wl,tokens,fused", [
    ("f32", _wl("tiny", seed=120), 64, False),
    ("bf16_fused", _wl("tiny", in_dtype="bf16", seed=121), 48, True),
    ("W20_two_launches", _wl("tiny", window=20, seed=122), 40, True),
    ("C8", _wl("tiny", n_comp=8, seed=123), 32, True),
    ("C0_nosmooth", _wl("tiny", n_comp=0, smoothing=False, seed=124), 20, False),
    ("ragged_heads", _wl("tiny", batch=3, heads=5, seed=125, init="prefill"), 32, True),
    ("hard", _wl("tiny", init="hard", batch=1, heads=32, seed=126), 33, True),
])
def test_low_bits_against_oracle(bits, name, wl, tokens, fused):
    progress(f"  case {name} at {bits} bits: {wl}")
    rep, L, _ = run_layer(wl, tokens=tokens, fused=fused, bits=bits)
    Q = L.codes().cpu().numpy()
    lv = 31 if bits == 6 else 7
    assert np.abs(Q.astype(np.int32)).max() <= lv
    _finish(rep)


@pytest.mark.parametrize("bits", [6, 4])
def test_low_bits_dequant_views(bits):
    wl = _wl("tiny", seed=127, init="prefill")
    H = wl.batch * wl.heads
    rep, L, refs = run_layer(wl, tokens=21, bits=bits)
    out = torch.empty(H, D, D, device="cuda")
    for what in (0, 1, 2):
        lq.leapq_dequant(L, what, out)
        got = out.cpu().numpy()
        for h in range(H):
            rep.fp(f"dequant{what}", got[h], refs[h].dequant(what))
    _finish(rep)


@pytest.mark.parametrize("bits", [6, 4])
def test_low_bits_edge_states(bits):
    """Exact .5 ties of the scaled values (codes picked from the fixture row's
    halves scaled to the level count), tiny and subnormal rows, and the
    fma-sensitive rebuild, each through a window and a fold."""
    rng = np.random.default_rng(128)
    lv = 31 if bits == 6 else 7
    # a row whose maximum is lv and whose other entries are exact halves
    S0 = np.zeros((3, D, D), np.float32)
    halves = np.array([lv, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5, lv - 0.5, -(lv - 0.5)], np.float32)
    for h, r in enumerate((9, 64, 127)):
        S0[h, r, :halves.size] = halves
        S0[h, r + 1 if r < 127 else 0] = (rng.standard_normal(D) * 0.01).astype(np.float32)
    tw = Twin(S0, C=0, smoothing=False, bits=bits)
    Q = tw.L.codes().cpu().numpy()
    want = np.rint(halves).astype(np.int32)  # ties to even
    for h, r in enumerate((9, 64, 127)):
        assert np.array_equal(Q[h, r, :halves.size].astype(np.int32), want), (h, Q[h, r, :halves.size])
    _finish(tw.rep)
    tw = Twin(edge.tiny_state(), C=4, smoothing=True, sigma_floor=1e-30, bits=bits)
    for t, tok in enumerate(edge._tokens(rng, 4, 16)):
        tw.append(tok, fused=t == 15)
    _finish(tw.rep)
    tw = Twin(edge.stress_state(), C=4, bits=bits)
    for tok in edge.stress_tokens(H=4):
        tw.append(tok)
    tw.fold()
    _finish(tw.rep)


@pytest.mark.parametrize("bits", [6, 4])
def test_low_bits_full_size_b512_sampled(bits):
    wl = WL["b512"]
    sample = list(range(11, 16384, 256))
    rep, _, _ = run_layer(wl, tokens=32, sample=sample, gen_device="cuda", check_every_token=False, fused=True,
                          bits=bits)
    _finish(rep)
