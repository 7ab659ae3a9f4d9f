"""Decode benchmark of the LeapQuant append + fold path on one MI355X.

One step = one window of the whole hot path: for each of the window's 16
tokens, the append of all 24 layers; each layer's 16th token and its fold run
as one leapq_append_fold call (--separate: append, then fold).
Workload (default "b512"): 24 GDN layers x 32 heads x 128x128 state, batch
512, W=16, C=4, bf16 q/k/v, fp32 records; seeded synthetic inputs (a pool of
16 tokens per layer, cycled every window), resident in HBM before timing.

Prints ONE JSON line on stdout; progress goes to stderr.

  python bench.py [--gpus 1] [--steps 64] [--warmup 2] [--workload b512]
                  [--no-baselines] [--no-cpu] [--separate]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tokens/s and HBM GB/s (% of peak), append+fold, 24Lx32H, batch 512"
HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "append_b512_traffic.json")
VALU_FILE = os.path.join(ROOT, "profiles", "append_fold_b512_valu.json")
# plain (unpacked) fp32 VALU issue rate: 256 CUs x 4 SIMDs x 16 lanes per
# cycle x 2.4 GHz, in lane-operations per second
VALU_PEAK_LANE_OPS = 256 * 4 * 16 * 2.4e9
N_SIMDS = 256 * 4
CLOCK_HZ = 2.4e9


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=64, help="timed windows (16 tokens each)")
    p.add_argument("--warmup", type=int, default=2, help="untimed windows")
    p.add_argument("--workload", default="b512")
    p.add_argument("--no-baselines", action="store_true")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--no-gated", action="store_true",
                   help="skip the gated-path measurement (gate arithmetic and q/k normalization in the append)")
    p.add_argument("--no-kda", action="store_true",
                   help="skip the per-channel decay (KDA) measurement at the same shape")
    p.add_argument("--no-bf16-records", action="store_true",
                   help="skip the measurement of the lossy bf16 record-corrections option")
    p.add_argument("--no-fp8-records", action="store_true",
                   help="skip the measurement of the lossy fp8 record-corrections option")
    p.add_argument("--no-low-bits", action="store_true",
                   help="skip the measurement of the 6- and 4-bit residual-state options")
    p.add_argument("--no-rank1", action="store_true",
                   help="skip the measurement of the rank-one compensator option")
    p.add_argument("--no-pattern", action="store_true",
                   help="skip the probe of the append's memory traffic without its arithmetic")
    p.add_argument("--no-block", action="store_true",
                   help="skip the measurement of the block compensator fit option")
    p.add_argument("--no-staggered", action="store_true",
                   help="skip the measurement of per-request window phases (leapq_step)")
    p.add_argument("--baseline-tokens", type=int, default=16)
    p.add_argument("--cpu-threads", type=int, default=16)
    p.add_argument("--separate", action="store_true",
                   help="leapq_append then leapq_fold for each window's last token (no fused call)")
    return p.parse_args()


def kernel_sha():
    from quantized_recurrent_state_amd.profiling import kernel_sha as sha
    return sha()


def fold_sha():
    from quantized_recurrent_state_amd.profiling import FOLD_SOURCES, kernel_sha as sha
    return sha(FOLD_SOURCES)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on one GPU only: every head is independent and the path has no "
              f"collective, so a multi-GPU run would only repeat this measurement per GPU "
              f"(requested --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from quantized_recurrent_state_amd import leapq as lq
    from quantized_recurrent_state_amd import metrics, profiling, workloads

    wl = workloads.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, Lyr, Hh, W, C = wl.batch, wl.layers, wl.heads, wl.window, wl.n_comp
    H = B * Hh
    D = 128
    in_bytes = 2 if wl.in_dtype == "bf16" else 4
    stream = torch.cuda.current_stream(dev)
    log(f"[bench] {wl.name}: {wl.notes}; {Lyr} layers x {H} heads; device {torch.cuda.get_device_name(0)}")

    # ---- state and inputs, resident before timing.  The initial states (512
    # prefill tokens of the dense fp32 recurrence per layer, then the outlier
    # lines) are built once and shared by every section below.
    t_pre = time.perf_counter()
    S0s = []
    for l in range(Lyr):
        S0s.append(workloads.initial_state(wl, l, device=dev).reshape(H, D, D))
        torch.cuda.synchronize(dev)
        log(f"[bench] initial state of layer {l + 1}/{Lyr} built "
            f"({workloads.PREFILL_TOKENS} prefill tokens, {time.perf_counter() - t_pre:.1f} s so far)")
    cfg = lq.make_config(B, Hh, W, C, wl.smoothing, wl.sigma_floor, wl.in_dtype)
    layers = []
    for l in range(Lyr):
        L = lq.Layer(cfg, dev)
        lq.leapq_init_state(L, S0s[l])
        layers.append(L)
    pool = []
    for l in range(Lyr):
        toks = []
        for pos in range(W):
            q, k, v, a, b = workloads.token_inputs(wl, l, pos, device=dev)
            toks.append((q.reshape(H, D), k.reshape(H, D), v.reshape(H, D), a.reshape(H), b.reshape(H)))
        pool.append(toks)
    outs = [torch.empty(H, D, dtype=torch.float32, device=dev) for _ in range(Lyr)]
    torch.cuda.synchronize(dev)
    log(f"[bench] states and input pool resident: "
        f"{torch.cuda.memory_allocated(dev) / 2**30:.1f} GiB allocated")

    def window(events=None, fused=True):
        """One window: W tokens through every layer.  With fused, each layer's
        last token and its fold are one leapq_append_fold call; otherwise
        leapq_append, then leapq_fold after the W-th token."""
        for pos in range(W):
            for l in range(Lyr):
                q, k, v, a, b = pool[l][pos]
                kind = "append_fold" if fused and layers[l].n_records == W - 1 else "append"
                if events is not None:
                    events.append((kind, pos, torch.cuda.Event(enable_timing=True)))
                    events[-1][2].record(stream)
                if kind == "append_fold":
                    lq.leapq_append_fold(layers[l], q, k, v, a, b, outs[l], stream)
                else:
                    lq.leapq_append(layers[l], q, k, v, a, b, outs[l], stream)
                if events is not None:
                    events.append(("end", pos, torch.cuda.Event(enable_timing=True)))
                    events[-1][2].record(stream)
                if layers[l].n_records == W:
                    if events is not None:
                        events.append(("fold", pos, torch.cuda.Event(enable_timing=True)))
                        events[-1][2].record(stream)
                    lq.leapq_fold(layers[l], stream)
                    if events is not None:
                        events.append(("end", pos, torch.cuda.Event(enable_timing=True)))
                        events[-1][2].record(stream)

    fused = not args.separate
    for _ in range(args.warmup):
        window(fused=fused)
    torch.cuda.synchronize(dev)
    log(f"[bench] warmup {args.warmup} windows done")

    # ---- timed region: K windows, bracketed by synchronize
    torch.cuda.synchronize(dev)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(stream)
    for s in range(args.steps):
        window(fused=fused)
        if (s + 1) % 16 == 0:
            log(f"[bench] timed windows enqueued: {s + 1}/{args.steps}")
    t1.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    ms_per_step = total_ms / args.steps
    tokens_per_s = B * W / (ms_per_step / 1e3)
    log(f"[bench] {args.steps} windows: {total_ms:.1f} ms on the GPU clock ({wall:.2f} s wall); "
        f"{ms_per_step:.3f} ms per window, {tokens_per_s:,.0f} tokens/s")

    # ---- per-launch durations (HIP events on the launch stream): 2 windows
    # of separate appends and folds, then 2 windows timing the fused launch
    ev_app = {pos: [] for pos in range(W)}
    ev_fold, ev_fused = [], []
    for mode in (False, False, True, True):
        events = []
        window(events, fused=mode)
        torch.cuda.synchronize(dev)
        for (kind, pos, e0), (_, _, e1) in zip(events[0::2], events[1::2]):
            dt = e0.elapsed_time(e1)
            if kind == "append_fold":
                ev_fused.append(dt)
            elif kind == "fold":
                ev_fold.append(dt)
            elif not mode:
                ev_app[pos].append(dt)
    app_us = {pos: 1e3 * float(np.mean(v)) for pos, v in ev_app.items()}
    # the plain appends of the timed schedule: positions 0..W-2 with the fused
    # last token, 0..W-1 without
    sched = list(range(W - 1)) if fused and W >= 2 else list(range(W))
    append_us = float(np.mean([app_us[p] for p in sched]))
    fold_us = 1e3 * float(np.mean(ev_fold))
    fused_us = 1e3 * float(np.mean(ev_fused)) if ev_fused else None
    app_bytes_avg = float(np.mean([metrics.append_bytes(n, C, in_bytes) for n in sched])) * H
    fold_bytes = metrics.fold_bytes(W, C, in_bytes) * H
    append_gbps = app_bytes_avg / (append_us * 1e-6) / 1e9
    fold_gbps = fold_bytes / (fold_us * 1e-6) / 1e9
    share_sep = metrics.fold_share(W * append_us, fold_us)
    # fused schedule: the fold's cost is what the fused launch adds to the
    # window's last append
    share = share_sep
    if fused and fused_us is not None and W >= 3:
        # the plain append at the last position, extrapolated from positions
        # 0..W-2: the measured one follows the previous layer's fold and
        # carries part of that fold's write-back
        last_app = float(np.polyval(np.polyfit(np.arange(W - 1), [app_us[p] for p in range(W - 1)], 1), W - 1))
        share = (fused_us - last_app) / (sum(app_us[p] for p in range(W - 1)) + fused_us)
    window_bytes = metrics.window_bytes(W, C, in_bytes) * H * Lyr
    path_gbps = window_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"[bench] append {append_us:.1f} us ({append_gbps:.0f} GB/s algorithmic), fold {fold_us:.1f} us "
        f"({fold_gbps:.0f} GB/s), last append + fold in one launch {fused_us:.1f} us; fold share "
        f"{100 * share:.1f}% ({100 * share_sep:.1f}% with a separate fold), whole path {path_gbps:.0f} GB/s")

    # the fused launch (the window's last append and the fold) against the
    # plain VALU issue rate: VALU instructions x 64 lanes per launch from the
    # recorded counters (while the kernels' sources are unchanged) over the
    # launch time measured here; matrix-core busy time beside it
    fold_roofline = {"bound": "alu", "kernel": "leapq append_fold (fused last append + fold)",
                     "achieved_gbps_algorithmic": fold_gbps, "peak": VALU_PEAK_LANE_OPS / 1e12,
                     "unit": "T lane-ops/s", "achieved": None, "frac": None}
    if os.path.exists(VALU_FILE) and fused_us:
        with open(VALU_FILE) as f:
            vc = json.load(f)
        if vc.get("kernel_sha") == fold_sha() and vc.get("workload") == wl.name:
            lane_ops = vc["insts_valu_per_launch"] * 64
            fold_roofline.update({
                "achieved": lane_ops / (fused_us * 1e-6) / 1e12,
                "frac": lane_ops / (fused_us * 1e-6) / VALU_PEAK_LANE_OPS,
                "valu_lane_ops_per_launch": lane_ops,
                "mfma_busy_frac": vc["mfma_busy_cycles_per_launch"] / (N_SIMDS * fused_us * 1e-6 * CLOCK_HZ),
                "mfma_valu_coexec_cycles_per_launch": vc.get("mfma_coexec_cycles_per_launch"),
                "counters": os.path.relpath(VALU_FILE, ROOT)})

    copy_gbps = copy_ceiling(torch, stream)
    log(f"[bench] streaming ceiling (1 GiB elementwise y = -x, 4 B read + 4 B written per element): "
        f"{copy_gbps:.0f} GB/s ({100 * copy_gbps / HBM_PEAK_GBPS:.1f}% of {HBM_PEAK_GBPS:.0f})")
    # the append's own loads and stores without its arithmetic (measurement
    # probe, four state copies in turn), and a plain streaming read of the
    # same bytes: the ceilings of this access pattern on this GPU
    pattern = None
    if not args.no_pattern and wl.decay == "scalar":
        pat = profiling.append_pattern(H, C, W, in_bytes, 4 * D, sched, reps=20)
        pat_us = float(np.mean([pat[p] for p in sched]))
        read_gbps = profiling.read_ceiling(int(app_bytes_avg), reps=20)
        pattern = {"us_mean": pat_us, "gbps": app_bytes_avg / (pat_us * 1e-6) / 1e9,
                   "us_by_position": [round(pat[p], 2) for p in sched],
                   "append_frac_of_pattern": pat_us / append_us,
                   "append_frac_of_pattern_by_position": [round(pat[p] / app_us[p], 3) for p in sched],
                   "read_ceiling_gbps": read_gbps}
        log(f"[bench] the append's memory traffic alone: {pat_us:.1f} us ({pattern['gbps']:.0f} GB/s); the "
            f"append runs at {100 * pattern['append_frac_of_pattern']:.1f}% of that rate; plain streaming read "
            f"of the same bytes {read_gbps:.0f} GB/s")

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_sha") == kernel_sha() and tr.get("workload") == wl.name:
            traffic = tr.get("bytes_per_launch")

    # ---- the gated path: raw projections in, gate arithmetic and q / k
    # normalization in the append (fp32 record keys), same schedule
    gated = None
    if not args.no_gated:
        gcfg = lq.make_config(B, Hh, W, C, wl.smoothing, wl.sigma_floor, wl.in_dtype, qk_norm=True)
        glayers, gpool, gates = [], [], []
        for l in range(Lyr):
            L = lq.Layer(gcfg, dev)
            lq.leapq_init_state(L, S0s[l])
            glayers.append(L)
            gates.append(lq.Gate(*workloads.gate_params(wl, l, device=dev)))
            toks = []
            for pos in range(W):
                q, k, v, a, b = workloads.gated_token_inputs(wl, l, pos, device=dev)
                toks.append((q.reshape(H, D), k.reshape(H, D), v.reshape(H, D), a.reshape(H), b.reshape(H)))
            gpool.append(toks)

        def gwindow(ev=None):
            for pos in range(W):
                for l in range(Lyr):
                    q, k, v, a, b = gpool[l][pos]
                    if ev is not None:
                        ev.append((pos, torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)))
                        ev[-1][1].record(stream)
                    if glayers[l].n_records == W - 1:
                        lq.leapq_append_fold_gated(glayers[l], gates[l], q, k, v, a, b, outs[l], stream)
                    else:
                        lq.leapq_append_gated(glayers[l], gates[l], q, k, v, a, b, outs[l], stream)
                    if ev is not None:
                        ev[-1][2].record(stream)

        gwindow()
        torch.cuda.synchronize(dev)
        gsteps = max(4, args.steps // 4)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(gsteps):
            gwindow()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        g_ms = e0.elapsed_time(e1) / gsteps
        gev = []
        gwindow(gev)
        torch.cuda.synchronize(dev)
        g_app = [1e3 * e0_.elapsed_time(e1_) for pos, e0_, e1_ in gev if pos < W - 1]
        g_fused = [1e3 * e0_.elapsed_time(e1_) for pos, e0_, e1_ in gev if pos == W - 1]
        gated = {"tokens_per_s": B * W / (g_ms / 1e3), "ms_per_step": g_ms, "steps": gsteps,
                 "ratio_to_plain": (B * W / (g_ms / 1e3)) / tokens_per_s,
                 "append_us": float(np.mean(g_app)), "append_fold_us": float(np.mean(g_fused)),
                 "inputs": "raw bf16 q/k/v and fp32 gate projections a, b; alpha, beta from A_log, dt_bias; "
                           "q, k L2-normalized in the append; fp32 record keys"}
        log(f"[bench] gated path: {g_ms:.3f} ms per window, {gated['tokens_per_s']:,.0f} tokens/s "
            f"({gated['ratio_to_plain']:.3f} of the plain path); append {gated['append_us']:.1f} us "
            f"(positions 0..{W - 2}), last append + fold {gated['append_fold_us']:.1f} us")
        del glayers, gpool, gates
        torch.cuda.empty_cache()

    # ---- layout options on the same inputs and schedule (separate
    # measurements, never the headline value)
    def time_option(vcfg, u_bytes=4, rank1=False, bits=8):
        vlayers = []
        for l in range(Lyr):
            L = lq.Layer(vcfg, dev)
            lq.leapq_init_state(L, S0s[l])
            vlayers.append(L)

        def vwindow(ev=None):
            for pos in range(W):
                for l in range(Lyr):
                    q, k, v, a, b = pool[l][pos]
                    if ev is not None:
                        ev.append((pos, torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)))
                        ev[-1][1].record(stream)
                    if vlayers[l].n_records == W - 1:
                        lq.leapq_append_fold(vlayers[l], q, k, v, a, b, outs[l], stream)
                    else:
                        lq.leapq_append(vlayers[l], q, k, v, a, b, outs[l], stream)
                    if ev is not None:
                        ev[-1][2].record(stream)

        vwindow()
        torch.cuda.synchronize(dev)
        vsteps = max(4, args.steps // 4)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(vsteps):
            vwindow()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        v_ms = e0.elapsed_time(e1) / vsteps
        vev = []
        vwindow(vev)
        torch.cuda.synchronize(dev)
        del vlayers
        torch.cuda.empty_cache()
        v_app = float(np.mean([1e3 * x.elapsed_time(y) for pos, x, y in vev if pos < W - 1]))
        v_bytes = float(np.mean([metrics.append_bytes(n, C, in_bytes, u_bytes=u_bytes, rank1=rank1, bits=bits)
                                 for n in range(W - 1)])) * H
        return {"tokens_per_s": B * W / (v_ms / 1e3), "ms_per_step": v_ms, "steps": vsteps,
                "ratio_to_plain": (B * W / (v_ms / 1e3)) / tokens_per_s, "append_us": v_app,
                "append_fold_us": float(np.mean([1e3 * x.elapsed_time(y) for pos, x, y in vev if pos == W - 1])),
                "append_gbps_algorithmic": v_bytes / (v_app * 1e-6) / 1e9}

    bf16rec = None
    if not args.no_bf16_records:
        bf16rec = time_option(lq.make_config(B, Hh, W, C, wl.smoothing, wl.sigma_floor, wl.in_dtype,
                                             rec_dtype="bf16"), u_bytes=2)
        bf16rec["note"] = "lossy option: record corrections rounded to bf16 (see quality.py --rec-dtype bf16)"
        log(f"[bench] bf16 record corrections: {bf16rec['ms_per_step']:.3f} ms per window, "
            f"{bf16rec['tokens_per_s']:,.0f} tokens/s ({bf16rec['ratio_to_plain']:.3f} of the plain path); "
            f"append {bf16rec['append_us']:.1f} us")

    fp8rec = None
    if not args.no_fp8_records:
        fp8rec = time_option(lq.make_config(B, Hh, W, C, wl.smoothing, wl.sigma_floor, wl.in_dtype,
                                            rec_dtype="fp8"), u_bytes=144 / 128)
        fp8rec["note"] = ("lossy option: record corrections as E4M3 with a power-of-two scale per 32 value columns "
                          "(see quality.py --rec-dtype fp8)")
        log(f"[bench] fp8 record corrections: {fp8rec['ms_per_step']:.3f} ms per window, "
            f"{fp8rec['tokens_per_s']:,.0f} tokens/s ({fp8rec['ratio_to_plain']:.3f} of the plain path); "
            f"append {fp8rec['append_us']:.1f} us")

    low_bits = {}
    if not args.no_low_bits:
        for bits in (6, 4):
            r = time_option(lq.make_config(B, Hh, W, C, wl.smoothing, wl.sigma_floor, wl.in_dtype, state_bits=bits),
                            bits=bits)
            r["note"] = (f"residual codes of {bits} bits (symmetric, {31 if bits == 6 else 7} levels), packed "
                         f"(see quality.py --state-bits {bits})")
            low_bits[f"{bits}_bit_state"] = r
            log(f"[bench] {bits}-bit residual state: {r['ms_per_step']:.3f} ms per window, "
                f"{r['tokens_per_s']:,.0f} tokens/s ({r['ratio_to_plain']:.3f} of the plain path); append "
                f"{r['append_us']:.1f} us ({r['append_gbps_algorithmic']:.0f} GB/s), last append + fold "
                f"{r['append_fold_us']:.1f} us")

    rank1 = None
    if not args.no_rank1:
        rank1 = time_option(lq.make_config(B, Hh, W, C, wl.smoothing, wl.sigma_floor, wl.in_dtype,
                                           comp_fit="rank1"), rank1=True)
        rank1["note"] = ("rank-one compensators fitted by power sweeps in the fold "
                         "(see quality.py --comp-fit rank1)")
        log(f"[bench] rank-one compensators: {rank1['ms_per_step']:.3f} ms per window, "
            f"{rank1['tokens_per_s']:,.0f} tokens/s ({rank1['ratio_to_plain']:.3f} of the plain path); "
            f"append {rank1['append_us']:.1f} us, last append + fold {rank1['append_fold_us']:.1f} us")

    block = None
    if not args.no_block:
        block = time_option(lq.make_config(B, Hh, W, C, wl.smoothing, wl.sigma_floor, wl.in_dtype,
                                           comp_fit="block"), rank1=True)
        block["note"] = ("compensator pairs fitted as a block, warm-started from the window's own pairs "
                         "(see quality.py --comp-fit block)")
        log(f"[bench] block compensator fit: {block['ms_per_step']:.3f} ms per window, "
            f"{block['tokens_per_s']:,.0f} tokens/s ({block['ratio_to_plain']:.3f} of the plain path); "
            f"append {block['append_us']:.1f} us, last append + fold {block['append_fold_us']:.1f} us")

    # ---- per-request window phases: request b is b % W tokens into its
    # window, so every step folds about 1/W of the requests (leapq_step, one
    # launch per layer and token); same inputs and work per window as the
    # lockstep schedule, with the fold spread over the window's tokens
    staggered = None
    if not args.no_staggered and W <= 16:
        slayers = []
        for l in range(Lyr):
            L = lq.Layer(cfg, dev)
            lq.leapq_init_state(L, S0s[l])
            slayers.append(L)
        ph = np.arange(B) % W
        # spread the phases: request b takes no token in the first W - ph[b] steps
        spread = [torch.as_tensor(np.where(t >= W - ph, t - (W - ph), -1).astype(np.int32), device=dev)
                  for t in range(W)]
        n_cur = torch.as_tensor(ph.astype(np.int32), device=dev)
        n_nxt = torch.empty_like(n_cur)

        def sstep(pos, n_in, n_out, ev=None):
            if ev is not None:
                ev.append(torch.cuda.Event(enable_timing=True))
                ev[-1].record(stream)
            for l in range(Lyr):
                q, k, v, a, b = pool[l][pos]
                lq.leapq_step(slayers[l], n_in, n_out, q, k, v, a, b, outs[l], stream=stream)
            if ev is not None:
                ev.append(torch.cuda.Event(enable_timing=True))
                ev[-1].record(stream)

        for t in range(W):
            sstep(t, spread[t], n_nxt)
        torch.cuda.synchronize(dev)
        # requests at phase 0 took no token (their n_out echoes -1)
        assert torch.equal(torch.where(n_cur > 0, n_nxt, n_cur), n_cur), "phase spread"

        def swindow(ev=None):
            nonlocal n_cur, n_nxt
            for pos in range(W):
                sstep(pos, n_cur, n_nxt, ev)
                n_cur, n_nxt = n_nxt, n_cur

        swindow()
        torch.cuda.synchronize(dev)
        ssteps = max(4, args.steps // 4)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(ssteps):
            swindow()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        s_ms = e0.elapsed_time(e1) / ssteps
        sev = []
        for _ in range(2):
            swindow(sev)
        torch.cuda.synchronize(dev)
        tok_ms = [x.elapsed_time(y) for x, y in zip(sev[0::2], sev[1::2])]
        lock_tok = [Lyr * app_us[p] / 1e3 for p in range(W - 1)] + [Lyr * fused_us / 1e3]
        staggered = {"tokens_per_s": B * W / (s_ms / 1e3), "ms_per_step": s_ms, "steps": ssteps,
                     "ratio_to_lockstep": (B * W / (s_ms / 1e3)) / tokens_per_s,
                     "token_ms_min": min(tok_ms), "token_ms_max": max(tok_ms),
                     "lockstep_token_ms_min": min(lock_tok), "lockstep_token_ms_max": max(lock_tok),
                     "phases": "request b at b % W tokens into its window"}
        log(f"[bench] per-request phases (leapq_step): {s_ms:.3f} ms per window, {staggered['tokens_per_s']:,.0f} "
            f"tokens/s ({staggered['ratio_to_lockstep']:.3f} of lockstep); one token through {Lyr} layers takes "
            f"{min(tok_ms):.3f}..{max(tok_ms):.3f} ms against {min(lock_tok):.3f}..{max(lock_tok):.3f} ms in lockstep")
        del slayers
        torch.cuda.empty_cache()

    # ---- per-channel decay (KDA): the same shape and schedule with alpha a
    # 128-vector per head and token, and the dense KDA baselines
    kda = None
    kname = wl.name + "_kda"
    if not args.no_kda and kname in workloads.WORKLOADS:
        kwl = workloads.WORKLOADS[kname]
        kcfg = lq.make_config(B, Hh, W, C, kwl.smoothing, kwl.sigma_floor, kwl.in_dtype, decay="channel")
        klayers, kpool, kS0s = [], [], []
        for l in range(Lyr):
            kS0s.append(workloads.initial_state(kwl, l, device=dev).reshape(H, D, D))
            L = lq.Layer(kcfg, dev)
            lq.leapq_init_state(L, kS0s[l])
            klayers.append(L)
            toks = []
            for pos in range(W):
                q, k, v, a, b = workloads.token_inputs(kwl, l, pos, device=dev)
                toks.append((q.reshape(H, D), k.reshape(H, D), v.reshape(H, D), a.reshape(H, D), b.reshape(H)))
            kpool.append(toks)

        def kwindow(ev=None):
            for pos in range(W):
                for l in range(Lyr):
                    q, k, v, a, b = kpool[l][pos]
                    if ev is not None:
                        ev.append((pos, torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)))
                        ev[-1][1].record(stream)
                    if klayers[l].n_records == W - 1:
                        lq.leapq_append_fold(klayers[l], q, k, v, a, b, outs[l], stream)
                    else:
                        lq.leapq_append(klayers[l], q, k, v, a, b, outs[l], stream)
                    if ev is not None:
                        ev[-1][2].record(stream)

        kwindow()
        torch.cuda.synchronize(dev)
        ksteps = max(4, args.steps // 4)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(ksteps):
            kwindow()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        k_ms = e0.elapsed_time(e1) / ksteps
        kev = []
        kwindow(kev)
        torch.cuda.synchronize(dev)
        k_app = [1e3 * e0_.elapsed_time(e1_) for pos, e0_, e1_ in kev if pos < W - 1]
        k_fused = [1e3 * e0_.elapsed_time(e1_) for pos, e0_, e1_ in kev if pos == W - 1]
        k_app_us = float(np.mean(k_app))
        k_bytes = float(np.mean([metrics.append_bytes(n, C, in_bytes, channel=True) for n in range(W - 1)])) * H
        kda = {"workload": f"{kwl.name}: {kwl.notes}", "tokens_per_s": B * W / (k_ms / 1e3), "ms_per_step": k_ms,
               "steps": ksteps, "append_us": k_app_us, "append_fold_us": float(np.mean(k_fused)),
               "append_gbps_algorithmic": k_bytes / (k_app_us * 1e-6) / 1e9,
               "hbm_gbps_path_algorithmic": metrics.window_bytes(W, C, in_bytes, channel=True) * H * Lyr
               / (k_ms * 1e-3) / 1e9}
        del klayers
        log(f"[bench] kda path: {k_ms:.3f} ms per window, {kda['tokens_per_s']:,.0f} tokens/s; append "
            f"{k_app_us:.1f} us ({kda['append_gbps_algorithmic']:.0f} GB/s algorithmic), last append + fold "
            f"{kda['append_fold_us']:.1f} us")
        if not args.no_baselines:
            for name, sdt, sbytes in (("fp32_state", torch.float32, 4), ("bf16_state", torch.bfloat16, 2)):
                states = [kS0s[l].to(sdt, copy=True).contiguous() for l in range(Lyr)]
                for pos in range(2):
                    for l in range(Lyr):
                        q, k, v, a, b = kpool[l][pos]
                        lq.leapq_gdn_decode(kcfg, states[l], q, k, v, a, b, outs[l], stream)
                torch.cuda.synchronize(dev)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                T = args.baseline_tokens
                e0.record(stream)
                for t in range(T):
                    for l in range(Lyr):
                        q, k, v, a, b = kpool[l][t % W]
                        lq.leapq_gdn_decode(kcfg, states[l], q, k, v, a, b, outs[l], stream)
                e1.record(stream)
                torch.cuda.synchronize(dev)
                ms_tok = e0.elapsed_time(e1) / T
                kgb = metrics.gdn_step_bytes(sbytes, in_bytes, channel=True) * H * Lyr / (ms_tok * 1e-3) / 1e9
                kda[name] = {"tokens_per_s": B / (ms_tok * 1e-3), "ms_per_token": ms_tok,
                             "hbm_gbps_algorithmic": kgb, "frac": kgb / HBM_PEAK_GBPS}
                kda[f"speedup_vs_{name}"] = kda["tokens_per_s"] / kda[name]["tokens_per_s"]
                log(f"[bench] kda baseline {name}: {ms_tok:.3f} ms/token, {B / (ms_tok * 1e-3):,.0f} tokens/s")
                del states
        del kpool, kS0s
        torch.cuda.empty_cache()

    # ---- baselines at the same shape: dense fp32-state and bf16-state decode
    baselines = None
    if not args.no_baselines:
        baselines = {}
        for name, sdt, sbytes in (("fp32_state", torch.float32, 4), ("bf16_state", torch.bfloat16, 2)):
            # the dense decode updates its state in place: a copy of each S0
            states = [S0s[l].to(sdt, copy=True).contiguous() for l in range(Lyr)]
            for pos in range(2):  # warmup
                for l in range(Lyr):
                    q, k, v, a, b = pool[l][pos]
                    lq.leapq_gdn_decode(cfg, states[l], q, k, v, a, b, outs[l], stream)
            torch.cuda.synchronize(dev)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            T = args.baseline_tokens
            e0.record(stream)
            for t in range(T):
                for l in range(Lyr):
                    q, k, v, a, b = pool[l][t % W]
                    lq.leapq_gdn_decode(cfg, states[l], q, k, v, a, b, outs[l], stream)
            e1.record(stream)
            torch.cuda.synchronize(dev)
            ms_tok = e0.elapsed_time(e1) / T
            gb = metrics.gdn_step_bytes(sbytes, in_bytes) * H * Lyr / (ms_tok * 1e-3) / 1e9
            baselines[name] = {"tokens_per_s": B / (ms_tok * 1e-3), "ms_per_token": ms_tok,
                               "hbm_gbps_algorithmic": gb, "frac": gb / HBM_PEAK_GBPS,
                               "frac_of_copy_ceiling": gb / copy_gbps}
            log(f"[bench] baseline {name}: {ms_tok:.3f} ms/token, {B / (ms_tok * 1e-3):,.0f} tokens/s, "
                f"{gb:.0f} GB/s")
            del states
            torch.cuda.empty_cache()

    # ---- CPU baseline: the oracle on one layer's heads for one window
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(wl, pool, S0s[0].cpu().numpy(), args.cpu_threads)

    result = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; 16-token input pool per layer, cycled every window)",
        "config": {"workload": f"{wl.name}: {wl.notes}", "batch": B, "layers": Lyr, "heads": Hh,
                   "dk": D, "dv": D, "window": W, "n_comp": C, "in_dtype": wl.in_dtype,
                   "state": "int8 residual + fp32 compensators + records (fp32 decays and corrections, keys in the input dtype)",
                   "tokens_per_step": W,
                   "schedule": ("W-1 appends + leapq_append_fold per layer and window" if fused
                                else "W appends + leapq_fold per layer and window")},
        "append_us": append_us,
        "append_positions": f"{sched[0]}..{sched[-1]} (the plain appends of the timed schedule)",
        "append_us_by_position": [round(app_us[p], 2) for p in range(W)],
        "fold_us": fold_us,
        "append_fold_us": fused_us,
        "fold_share": share,
        "fold_share_separate_fold": share_sep,
        "hbm_gbps_path_algorithmic": path_gbps,
        "roofline": {"bound": "hbm", "kernel": "leapq append", "achieved": append_gbps,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": append_gbps / HBM_PEAK_GBPS,
                     "traffic": traffic,
                     "bytes_per_launch_algorithmic": app_bytes_avg,
                     "copy_ceiling_gbps": copy_gbps, "frac_of_copy_ceiling": append_gbps / copy_gbps,
                     "pattern_ceiling": pattern},
        "fold_roofline": fold_roofline,
        "gated": gated,
        "kda": kda,
        "bf16_record_corrections": bf16rec,
        "fp8_record_corrections": fp8rec,
        "low_bit_states": low_bits or None,
        "rank1_compensators": rank1,
        "block_compensators": block,
        "staggered_phases": staggered,
        "baselines": baselines,
        "cpu_baseline": cpu,
        "kernel_sha": kernel_sha(),
    }
    if baselines:
        result["speedup_vs_fp32_state"] = tokens_per_s / baselines["fp32_state"]["tokens_per_s"]
        result["speedup_vs_bf16_state"] = tokens_per_s / baselines["bf16_state"]["tokens_per_s"]
    print(json.dumps(result), flush=True)


def copy_ceiling(torch, stream, mib=1024, reps=8):
    """GB/s of a plain elementwise kernel over `mib` MiB of fp32 (one read and
    one write per element), events on the launch stream: the streaming rate
    this GPU sustains in practice, beside the 8 TB/s of the data sheet."""
    n = mib * 2**20 // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.neg(x, out=y)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        torch.neg(x, out=y)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del x, y
    return 2 * n * 4 / (ms * 1e-3) / 1e9


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(wl, pool, S0, threads):
    """The oracle (unmodified, single-threaded per head; heads spread over a
    thread pool) on layer 0's heads for one whole window, scaled to the
    workload's tokens/s."""
    import concurrent.futures as cf

    import numpy as np

    import oracle

    H = wl.batch * wl.heads
    toks = [tuple(x.float().cpu().numpy() for x in pool[0][pos]) for pos in range(wl.window)]
    heads = list(range(H))

    def one(h):
        st = oracle.Head(wl.n_comp, wl.window, wl.smoothing, wl.sigma_floor).init(S0[h])
        for (q, k, v, a, b) in toks:
            st.append(q[h], k[h], v[h], a[h], b[h])
        st.fold()
        return 1

    oracle.lib()
    log(f"[bench] cpu baseline: oracle on {H} heads x 1 window, {threads} threads")
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        done = 0
        for i, _ in enumerate(ex.map(one, heads)):
            done += 1
            if done % 4096 == 0:
                log(f"[bench] cpu baseline heads done: {done}/{H}")
    dt = time.perf_counter() - t0
    scale = wl.layers  # one layer of the workload's layers
    tok_s = wl.batch * wl.window / (dt * scale)
    log(f"[bench] cpu baseline: {dt:.2f} s for one layer-window -> {tok_s:.1f} tokens/s")
    return {"value": tok_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"layer 0 only ({H} heads), one window (16 appends + fold per head), "
                      f"{dt:.2f} s wall; scaled by {scale} layers (a bounded sample: the full "
                      f"{scale}-layer window would hold the run for about {dt * scale / 60:.0f} minutes)",
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}


if __name__ == "__main__":
    main()
