"""GPU parity of the fp8 record corrections option (rec_dtype = fp8)
through the C ABI.

Each record's corrections are stored as OCP E4M3 codes with one power-of-two
scale per group of 32 value columns (the token that makes the record reads
out with its fp32 value); later reads and the fold use the stored value.
Runs are free-running against the oracle's rec_u="fp8" heads with the bar of
tests/gpu_harness.py, bitwise on every fp32 value; the GPU's stored codes
are decoded with torch's float8_e4m3fn for the comparison.
"""
import dataclasses

import numpy as np
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
    ("f32", _wl("tiny", seed=90), 64, False),
    ("bf16_fused", _wl("tiny", in_dtype="bf16", seed=91), 48, True),
    ("W20_two_launches", _wl("tiny", window=20, seed=92), 40, True),
    ("W64", _wl("tiny", window=64, seed=93, init="prefill"), 64, False),
    ("C8", _wl("tiny", n_comp=8, seed=94), 32, True),
    ("ragged_heads", _wl("tiny", batch=3, heads=5, seed=95), 32, True),
    ("hard", _wl("tiny", init="hard", batch=1, heads=32, seed=96), 33, True),
])
def test_fp8_records_against_oracle(name, wl, tokens, fused):
    progress(f"  case {name}: {wl}")
    rep, L, _ = run_layer(wl, tokens=tokens, fused=fused, rec_u="fp8")
    assert L.n_records == tokens % wl.window
    codes, scales = L.rec_u_physical()
    assert codes.dtype == torch.uint8 and scales.shape[-1] == 4
    if L.n_records:
        s = scales[:, :L.n_records].cpu().numpy()
        m, e = np.frexp(s)
        assert np.all(m == 0.5), "record scales are powers of two"
    _finish(rep)


def test_fp8_records_dequant_current():
    wl = _wl("tiny", seed=97, init="prefill")
    H = wl.batch * wl.heads
    rep, L, refs = run_layer(wl, tokens=23, rec_u="fp8")
    out = torch.empty(H, D, D, device="cuda")
    lq.leapq_dequant(L, lq.LEAPQ_DEQ_CURRENT, out)
    got = out.cpu().numpy()
    for h in range(H):
        rep.fp("dequant2", got[h], refs[h].dequant(2))
    _finish(rep)


def test_fp8_records_full_size_b512_sampled():
    wl = WL["b512"]
    sample = list(range(5, 16384, 256))
    rep, _, _ = run_layer(wl, tokens=32, sample=sample, gen_device="cuda", check_every_token=False, fused=True,
                          rec_u="fp8")
    _finish(rep)
