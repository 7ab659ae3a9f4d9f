"""Smoothing-axis study on the long workload, on the CPU with the oracle only.

"LeapQuant" 3.4 describes the residual smoothing as a rescaling of the key
rows (its inverse restores the key coordinates); the path built here smooths
per value column and keeps its int8 scales per key row.  This script measures
both readings on the long workload's first layer (8 requests x 32 heads; heads
24..31 of each request slowly decaying with x200 outlier lines), 4,095 tokens.

Each head runs the dense fp32 recurrence (the oracle's dense step) three ways:
unquantized (the reference), and with the state replaced by its quantized
boundary state (lines, smoothing, int8, then dequantized) at the start and
after every 16th token, once with each smoothing axis.  Within a window the
windowed path equals the dense recurrence from its boundary up to fp32
rounding (pinned by the oracle's window_vs_dense pins), so this reproduces the
error of the windowed path; the script also runs the windowed oracle itself
(value axis) on a few heads and prints both errors side by side.

Error per head: ||O - O_ref||_F / ||O_ref||_F over all tokens' outputs.

    python -m tests.study_smoothing_axis [--tokens 4095] [--threads 8]
"""
import argparse
import concurrent.futures as cf
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from quantized_recurrent_state_amd import workloads  # noqa: E402

D = 128


def summary(err, mask):
    e = np.asarray(err)[mask]
    return {"median": float(np.median(e)), "p90": float(np.percentile(e, 90)), "max": float(np.max(e)),
            "heads": int(mask.sum())}


def main(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--tokens", type=int, default=4095)
    p.add_argument("--threads", type=int, default=min(16, os.cpu_count() or 4))
    p.add_argument("--windowed-heads", type=int, nargs="*", default=[0, 5, 24, 29])
    a = p.parse_args(argv)
    wl = workloads.WORKLOADS["long"]
    H = wl.batch * wl.heads
    W, C = wl.window, wl.n_comp
    L = oracle.lib()
    t0 = time.perf_counter()
    S0 = workloads.initial_state(wl, 0).reshape(H, D, D).numpy()
    print(f"[study] initial states of {H} heads ready in {time.perf_counter() - t0:.1f} s", flush=True)
    hard = np.array([h % wl.heads >= 24 for h in range(H)])

    def snap(S, axis):
        return oracle.quantize_axis(S, C, wl.smoothing, wl.sigma_floor, axis=axis, L=L)[5]

    ref = [S0[h].copy() for h in range(H)]
    run = {ax: [snap(S0[h], ax) for h in range(H)] for ax in ("value", "key")}
    wh = list(a.windowed_heads)
    win = [oracle.Head(C, W, wl.smoothing, wl.sigma_floor, L=L).init(S0[h]) for h in wh]
    num = {ax: np.zeros(H) for ax in run}
    num["windowed"] = np.zeros(len(wh))
    den = np.zeros(H)

    def step_head(h, tok, fold):
        q, k, v, al, be = (x[h] for x in tok)
        _, o_ref = oracle.gdn_step_f32(ref[h], q, k, v, al, be, L=L)
        den[h] += float(np.sum(o_ref.astype(np.float64) ** 2))
        for ax, states in run.items():
            _, o = oracle.gdn_step_f32(states[h], q, k, v, al, be, L=L)
            num[ax][h] += float(np.sum((o.astype(np.float64) - o_ref) ** 2))
            if fold:
                states[h] = snap(states[h], ax)
        return o_ref

    with cf.ThreadPoolExecutor(max_workers=a.threads) as ex:
        for t in range(a.tokens):
            q, k, v, al, be = workloads.token_inputs(wl, 0, t)
            tok = (q.reshape(H, D).numpy(), k.reshape(H, D).numpy(), v.reshape(H, D).numpy(),
                   al.reshape(H).numpy(), be.reshape(H).numpy())
            fold = (t + 1) % W == 0
            outs = list(ex.map(lambda h: step_head(h, tok, fold), range(H)))
            for j, h in enumerate(wh):
                o, _ = win[j].append(*(x[h] for x in tok))
                num["windowed"][j] += float(np.sum((o.astype(np.float64) - outs[h]) ** 2))
                if fold:
                    win[j].fold()
            if (t + 1) % 256 == 0:
                print(f"[study] token {t + 1}/{a.tokens} ({time.perf_counter() - t0:.0f} s)", flush=True)
    err = {ax: np.sqrt(num[ax] / den) for ax in ("value", "key")}
    res = {"workload": f"long layer 0 ({H} heads), {a.tokens} tokens, W = {W}, C = {C}",
           "value_axis (built)": {"regular": summary(err["value"], ~hard), "hard": summary(err["value"], hard)},
           "key_axis (study)": {"regular": summary(err["key"], ~hard), "hard": summary(err["key"], hard)},
           "check: windowed oracle vs snapped recurrence, value axis, heads": {
               str(h): [float(np.sqrt(num["windowed"][j] / den[h])), float(err["value"][h])]
               for j, h in enumerate(wh)}}
    print(json.dumps(res, indent=1))
    return res


if __name__ == "__main__":
    main()
