"""Long-horizon error of the quantized state against unquantized references.

For every head of a workload this runs, token by token on the GPU:
  - the LeapQuant path (append every token, fold after every W-th),
  - the fp32-state GDN recurrence from the unquantized initial state,
  - a bf16 state updated in fp32 and rounded to nearest even every token,
and reports per head the output error ||O - O_ref||_F / ||O_ref||_F over all
tokens and value columns, with the fp32 recurrence as O_ref ("LeapQuant:
Efficient Linear Attention with Accurate Recurrent State Quantization", 1
Introduction: a state rounded every step compounds its error; 3.2: rounding
once per window keeps it bounded).  Heads are summarized separately for the
regular heads and the hard heads of the "long" workload (slow decay, heavy
outliers).  With per-channel decay ("long_kda") the references are the
fp32-state and bf16-state KDA recurrences.

A caller may pass `on_token(layer, t, inputs, o, folded)`, called after every
token with that token's inputs (q, k, v, alpha, beta as handed to the GPU),
the GPU output and whether a fold followed; the parity tests use it to run
CPU reference heads beside the GPU path.

  python -m quantized_recurrent_state_amd.quality [--workload long] [--layers 3]
         [--tokens 4095] [--rec-dtype f32|bf16|fp8] [--comp-fit lines|rank1|block] [--state-bits 8|6|4]
         [--out result.json]
"""
import argparse
import json
import sys
import time

import numpy as np
import torch

from . import leapq as lq
from . import workloads

D = 128


def _summ(x):
    x = np.sort(np.asarray(x, np.float64))
    if x.size == 0:
        return None
    return {"median": float(np.median(x)), "p90": float(np.quantile(x, 0.9)), "max": float(x[-1]),
            "heads": int(x.size)}


def run(workload="long", layers=None, tokens=None, device="cuda:0", log=print, on_token=None, rec_dtype="f32",
        comp_fit="lines", state_bits=8):
    wl = workloads.WORKLOADS[workload]
    dev = torch.device(device)
    B, Hh, W, C = wl.batch, wl.heads, wl.window, wl.n_comp
    H = B * Hh
    nlayers = wl.layers if layers is None else layers
    T = wl.tokens if tokens is None else tokens
    cfg = lq.make_config(B, Hh, W, C, wl.smoothing, wl.sigma_floor, wl.in_dtype, decay=wl.decay, rec_dtype=rec_dtype,
                         comp_fit=comp_fit, state_bits=state_bits)
    ash = (H, D) if wl.decay == "channel" else (H,)
    rel_q, rel_b, hard = [], [], []
    for layer in range(nlayers):
        S0 = workloads.initial_state(wl, layer, device=dev).reshape(H, D, D).contiguous()
        L = lq.Layer(cfg, dev)
        lq.leapq_init_state(L, S0)
        S32 = S0.clone()
        S16 = S0.to(torch.bfloat16).contiguous()
        oq = torch.empty(H, D, dtype=torch.float32, device=dev)
        o32 = torch.empty_like(oq)
        o16 = torch.empty_like(oq)
        eq = torch.zeros(H, dtype=torch.float64, device=dev)
        eb = torch.zeros_like(eq)
        r2 = torch.zeros_like(eq)
        t0 = time.perf_counter()
        for t in range(T):
            q, k, v, a, b = workloads.token_inputs(wl, layer, t, device=dev)
            q, k, v = q.reshape(H, D), k.reshape(H, D), v.reshape(H, D)
            a, b = a.reshape(ash), b.reshape(H)
            lq.leapq_append(L, q, k, v, a, b, oq)
            lq.leapq_gdn_decode(cfg, S32, q, k, v, a, b, o32)
            lq.leapq_gdn_decode(cfg, S16, q, k, v, a, b, o16)
            ref = o32.double()
            eq += (oq.double() - ref).square().sum(-1)
            eb += (o16.double() - ref).square().sum(-1)
            r2 += ref.square().sum(-1)
            folded = L.n_records == W
            if folded:
                lq.leapq_fold(L)
            if on_token is not None:
                on_token(layer, t, (q, k, v, a, b), oq, folded)
            if (t + 1) % 1024 == 0:
                torch.cuda.synchronize(dev)
                log(f"[quality] {wl.name} layer {layer}: token {t + 1}/{T} ({time.perf_counter() - t0:.1f} s)")
        rq = torch.sqrt(eq / r2).cpu().numpy()
        rb = torch.sqrt(eb / r2).cpu().numpy()
        hh = np.arange(H) % Hh
        is_hard = (hh >= 24) if wl.init == "hard" else np.zeros(H, bool)
        rel_q.append(rq)
        rel_b.append(rb)
        hard.append(is_hard)
        del L, S32, S16
    rq, rb, hd = np.concatenate(rel_q), np.concatenate(rel_b), np.concatenate(hard)
    out = {
        "workload": wl.name, "layers": nlayers, "tokens": T, "heads_per_layer": H, "record_corrections": rec_dtype,
        "compensators": comp_fit, "state_bits": state_bits,
        "metric": "per-head ||O - O_fp32||_F / ||O_fp32||_F over all tokens",
        "leapq": {"regular": _summ(rq[~hd]), "hard": _summ(rq[hd])},
        "bf16_per_token": {"regular": _summ(rb[~hd]), "hard": _summ(rb[hd])},
        "finite": bool(np.all(np.isfinite(rq)) and np.all(np.isfinite(rb))),
    }
    return out


def main(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--workload", default="long")
    p.add_argument("--layers", type=int, default=None)
    p.add_argument("--tokens", type=int, default=None)
    p.add_argument("--rec-dtype", default="f32", choices=("f32", "bf16", "fp8"),
                   help="storage of the record corrections (bf16, fp8: the lossy lower-precision options)")
    p.add_argument("--comp-fit", default="lines", choices=("lines", "rank1", "block"),
                   help="compensator fit: whole rows/columns, rank-one pairs from power sweeps, or pairs "
                        "fitted as a block warm-started from the previous window")
    p.add_argument("--state-bits", type=int, default=8, choices=(8, 6, 4),
                   help="bits per residual code (6 and 4: the lower-precision state options)")
    p.add_argument("--out", default=None)
    a = p.parse_args(argv)
    res = run(a.workload, a.layers, a.tokens, log=lambda m: print(m, file=sys.stderr, flush=True),
              rec_dtype=a.rec_dtype, comp_fit=a.comp_fit, state_bits=a.state_bits)
    s = json.dumps(res, indent=1)
    print(s, flush=True)
    if a.out:
        with open(a.out, "w") as f:
            f.write(s + "\n")


if __name__ == "__main__":
    main()
