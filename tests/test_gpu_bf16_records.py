"""GPU parity of the bf16 record corrections option (rec_dtype = bf16)
through the C ABI.

The stored correction of each record is rounded to nearest even in bf16 (the
token that makes it reads out with the fp32 value); later reads and the fold
use the stored value.  Runs are free-running against the oracle's rec_u="bf16"
heads with the bar of tests/gpu_harness.py, bitwise on every fp32 value.
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


@pytest.mark.parametrize("name,wl,tokens,fused", [
    ("f32", _wl("tiny", seed=80), 64, False),
    ("bf16_fused", _wl("tiny", in_dtype="bf16", seed=81), 48, True),
    ("W20_two_launches", _wl("tiny", window=20, seed=82), 40, True),
    ("W64", _wl("tiny", window=64, seed=83, init="prefill"), 64, False),
    ("C8", _wl("tiny", n_comp=8, seed=84), 32, True),
    ("ragged_heads", _wl("tiny", batch=3, heads=5, seed=85), 32, True),
])
def test_bf16_records_against_oracle(name, wl, tokens, fused):
    progress(f"  case {name}: {wl}")
    rep, L, _ = run_layer(wl, tokens=tokens, fused=fused, rec_u="bf16")
    assert L.n_records == tokens % wl.window
    assert L.rec_u_physical().dtype == torch.bfloat16
    _finish(rep)


def test_bf16_records_dequant_current():
    wl = _wl("tiny", seed=86, init="prefill")
    H = wl.batch * wl.heads
    rep, L, refs = run_layer(wl, tokens=23, rec_u="bf16")
    out = torch.empty(H, D, D, device="cuda")
    lq.leapq_dequant(L, lq.LEAPQ_DEQ_CURRENT, out)
    got = out.cpu().numpy()
    for h in range(H):
        rep.fp("dequant2", got[h], refs[h].dequant(2))
    _finish(rep)


def test_bf16_records_full_size_b512_sampled():
    wl = WL["b512"]
    sample = list(range(3, 16384, 256))
    rep, _, _ = run_layer(wl, tokens=32, sample=sample, gen_device="cuda", check_every_token=False, fused=True,
                          rec_u="bf16")
    _finish(rep)
