"""GPU parity of the gated entry points (gate arithmetic fused in front of the
append) through the C ABI.

The GPU takes the raw projections (workloads.gated_token_inputs) and the
layer's gate parameters; the oracle applies oracle.gated_inputs (binary64
gates rounded once, fp32 L2 normalization) and then its append.  Runs are
free-running with the bar of tests/gpu_harness.py; the record decays compare
the gated alpha bit for bit, the record keys the normalized k.  One case runs
the plain leapq_append on a layer whose keys are fp32 because it normalizes
(bf16 inputs widened into fp32 keys).
"""
import dataclasses

import pytest

from quantized_recurrent_state_amd import workloads
from tests.gpu_harness import progress, run_layer

pytestmark = pytest.mark.gpu

WL = workloads.WORKLOADS
G = dict(q_scale=128 ** -0.5, eps=1e-6)


def _wl(base, **kw):
    return dataclasses.replace(WL[base], **kw)


def _finish(rep):
    progress(f"    summary: {rep.summary()}")
    rep.check()
    assert sum(rep.nonbit.values()) == 0, rep.nonbit


@pytest.mark.parametrize("name,wl,tokens,fused,qk_norm", [
    ("f32_norm", WL["tiny"], 48, False, True),
    ("f32_norm_fused", _wl("tiny", seed=50), 48, True, True),
    ("bf16_norm_fused", _wl("tiny", in_dtype="bf16", seed=51), 48, True, True),
    ("bf16_gates_only", _wl("tiny", in_dtype="bf16", seed=52), 40, True, False),
    ("f32_gates_only", _wl("tiny", seed=53), 20, False, False),
    ("ragged_heads", _wl("tiny", batch=3, heads=5, seed=54), 32, True, True),
    ("W20_two_launches", _wl("tiny", window=20, seed=55), 40, True, True),
])
def test_gated_against_oracle(name, wl, tokens, fused, qk_norm):
    progress(f"  case {name}: {wl}")
    rep, L, _ = run_layer(wl, tokens=tokens, fused=fused, gated=G, qk_norm=qk_norm)
    assert L.n_records == tokens % wl.window
    _finish(rep)


def test_plain_append_on_fp32_key_layer():
    """bf16 inputs, fp32 record keys (a layer set up for normalizing appends)
    driven by the plain entry points: the keys are the widened inputs."""
    wl = _wl("tiny", in_dtype="bf16", seed=56)
    rep, L, _ = run_layer(wl, tokens=40, fused=True, qk_norm=True)
    assert L.key_dtype.is_floating_point and L.rec_k_physical().element_size() == 4
    _finish(rep)


def test_gated_full_size_b512_every_head():
    """A whole gated, normalizing b512 layer, every head in the oracle: one
    window in the benchmark's schedule, all outputs and, after the fold, the
    whole boundary state bit for bit."""
    wl = WL["b512"]
    rep, _, _ = run_layer(wl, tokens=wl.window, sample=None, gen_device="cuda", check_every_token=False,
                          fused=True, gated=G, qk_norm=True)
    _finish(rep)


def test_gated_full_size_b512_sampled():
    """The benchmark's launch shape, gated and normalized: 64 sampled heads
    through 2 windows, the fused last token included."""
    wl = WL["b512"]
    sample = list(range(5, 16384, 256))
    rep, _, _ = run_layer(wl, tokens=32, sample=sample, gen_device="cuda", check_every_token=False, fused=True,
                          gated=G, qk_norm=True)
    _finish(rep)
