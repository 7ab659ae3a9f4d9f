"""Short GPU programs for rocprofv3 runs, and the reduction of its CSV output.

Programs (each is what comes after `rocprofv3 ... --`):

  python3 -m quantized_recurrent_state_amd.profiling run [--workload b512] [--windows 2] [--fused]
      one layer of the workload: init, then `windows` x (W appends + fold), or
      with --fused x (W-1 appends + the last append and fold in one launch)
  python3 -m quantized_recurrent_state_amd.profiling copy [--mib 1024] [--reps 4]
      a copy-shaped elementwise kernel (y = -x: 4 bytes read and 4 written
      per element; torch's same-dtype copy_ is a DMA blit, not a kernel) of
      known size, to calibrate FETCH_SIZE and WRITE_SIZE against bytes moved
  python3 -m quantized_recurrent_state_amd.profiling coexec [--agpr] [--lds 40960] [--reps 10]
      matrix-step / VALU co-execution probe: all-matrix, all-VALU and half/half
      launches (libleapq_probe.so, or with --agpr libleapq_probe_agpr.so)
  python3 -m quantized_recurrent_state_amd.profiling pattern [--workload b512] [--reps 20]
      the append's memory traffic alone (libleapq_probe.so: the append's
      loads and stores in the state layout, no arithmetic) at every window
      position, and a plain streaming read of the same bytes; one JSON object

Reductions (CPU only, read the CSV files rocprofv3 wrote):

  python3 -m quantized_recurrent_state_amd.profiling traffic \
      --kernel 'k_append<' --fetch F.csv --write W.csv \
      --copy-fetch CF.csv --copy-write CW.csv --copy-mib 1024 --workload b512 --out X.json
  python3 -m quantized_recurrent_state_amd.profiling stats --csv kernel_stats.csv
  python3 -m quantized_recurrent_state_amd.profiling valu --kernel k_append_fold \
      --csv SQ.csv [--csv SQ2.csv] --workload b512 --out X.json
      VALU instructions, waves and matrix-core busy cycles per launch from
      SQ_INSTS_VALU, SQ_WAVES, SQ_VALU_MFMA_BUSY_CYCLES (and, when present,
      SQ_VALU_MFMA_COEXEC_CYCLES, SQ_INSTS_MFMA) counter runs
"""
import argparse
import ctypes
import csv
import hashlib
import json
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
D = 128


# the sources of the append kernel: its traffic figure holds while they are unchanged
APPEND_SOURCES = ("leapq_append.hip", "leapq_append_dev.h", "leapq_device.h")
# the sources of the fold kernels (the fused last append + fold includes the append's)
FOLD_SOURCES = ("leapq_fold.hip", "leapq_append_dev.h", "leapq_device.h")


def kernel_sha(srcs=APPEND_SOURCES):
    h = hashlib.sha256()
    for src in srcs:
        with open(os.path.join(PKG, "csrc", src), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------- programs
def run_layer(workload, windows, fused=False):
    import torch

    from . import leapq as lq
    from . import workloads

    wl = workloads.WORKLOADS[workload]
    dev = torch.device("cuda:0")
    H, D = wl.batch * wl.heads, 128
    toks = []
    for pos in range(wl.window):
        q, k, v, a, b = workloads.token_inputs(wl, 0, pos, device=dev)
        toks.append((q.reshape(H, D), k.reshape(H, D), v.reshape(H, D), a.reshape(H), b.reshape(H)))
    S0 = workloads.initial_state(wl, 0, device=dev).reshape(H, D, D)
    o = torch.empty(H, D, dtype=torch.float32, device=dev)
    L = lq.Layer(lq.make_config(wl.batch, wl.heads, wl.window, wl.n_comp, wl.smoothing,
                                wl.sigma_floor, wl.in_dtype), dev)
    lq.leapq_init_state(L, S0)
    for w in range(windows):
        for n in range(wl.window):
            q, k, v, a, b = toks[n]
            if fused and n == wl.window - 1:
                lq.leapq_append_fold(L, q, k, v, a, b, o)
            else:
                lq.leapq_append(L, q, k, v, a, b, o)
        if not fused:
            lq.leapq_fold(L)
        torch.cuda.synchronize(dev)
        print(f"[profiling] {wl.name} layer 0: window {w + 1}/{windows} done", flush=True)


def run_copy(mib, reps):
    import torch

    n = mib * 2**20 // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    for r in range(reps):
        torch.neg(x, out=y)  # an elementwise kernel: one read and one write per element
    torch.cuda.synchronize()
    print(f"[profiling] copy {mib} MiB x {reps} done", flush=True)


_PROBE = {}


def probe_lib(agpr=False):
    """libleapq_probe.so, or with agpr libleapq_probe_agpr.so (built beside
    libleapq.so).  Raises if it is missing."""
    if agpr not in _PROBE:
        from . import build as _build

        path = _build.PROBE_LIB_AGPR if agpr else _build.PROBE_LIB
        if not os.path.exists(path):
            raise RuntimeError(f"{path} not found; run __graft_entry__.build()")
        L = ctypes.CDLL(path)
        i32 = ctypes.c_int
        L.lqp_append_pattern.argtypes = [i32, i32, i32, i32, i32, i32, i32, ctypes.POINTER(ctypes.c_float)]
        L.lqp_append_pattern.restype = i32
        L.lqp_read_ceiling.argtypes = [ctypes.c_size_t, i32, ctypes.POINTER(ctypes.c_float)]
        L.lqp_read_ceiling.restype = i32
        L.lqp_coexec.argtypes = [i32, i32, i32, ctypes.POINTER(ctypes.c_float)]
        L.lqp_coexec.restype = i32
        _PROBE[agpr] = L
    return _PROBE[agpr]


def coexec(agpr=False, lds=40960, reps=10):
    """Microseconds per launch of the co-execution probe: {mode: us} for
    mode 0 (all matrix steps), 1 (all VALU), 2 (half and half)."""
    out = {}
    for mode in (0, 1, 2):
        us = ctypes.c_float()
        rc = probe_lib(agpr).lqp_coexec(mode, lds, reps, ctypes.byref(us))
        if rc != 0:
            raise RuntimeError(f"lqp_coexec(mode={mode}) failed with HIP error {rc}")
        out[mode] = float(us.value)
    return out


def run_coexec(agpr, lds, reps):
    t = coexec(agpr, lds, reps)
    res = {"accumulators": "AGPR" if agpr else "VGPR", "lds_bytes_per_workgroup": lds, "workgroups": 16384,
           "us_all_matrix": t[0], "us_all_valu": t[1], "us_half_half": t[2],
           "us_halves_in_turn": (t[0] + t[1]) / 2, "us_halves_overlapped": max(t[0], t[1]) / 2}
    print(json.dumps(res), flush=True)
    return res


def append_pattern(heads, C, W, in_bytes, u_bytes, positions, reps=20):
    """Mean microseconds per launch of the append's memory traffic alone, at
    each record count n in `positions`: {n: us}."""
    out = {}
    for n in positions:
        us = ctypes.c_float()
        rc = probe_lib().lqp_append_pattern(heads, C, W, in_bytes, u_bytes, n, reps, ctypes.byref(us))
        if rc != 0:
            raise RuntimeError(f"lqp_append_pattern(n={n}) failed with HIP error {rc}")
        out[n] = float(us.value)
    return out


def read_ceiling(nbytes, reps=20):
    """GB/s of a plain streaming read of `nbytes` (four buffers in turn)."""
    us = ctypes.c_float()
    rc = probe_lib().lqp_read_ceiling(int(nbytes), reps, ctypes.byref(us))
    if rc != 0:
        raise RuntimeError(f"lqp_read_ceiling failed with HIP error {rc}")
    return nbytes / (us.value * 1e-6) / 1e9


def run_pattern(workload, reps):
    from . import metrics, workloads

    wl = workloads.WORKLOADS[workload]
    H, W, C = wl.batch * wl.heads, wl.window, wl.n_comp
    in_bytes = 2 if wl.in_dtype == "bf16" else 4
    pos = list(range(W - 1))
    t = append_pattern(H, C, W, in_bytes, 4 * D, pos, reps)
    by = {n: metrics.append_bytes(n, C, in_bytes) * H for n in pos}
    mean_us = sum(t.values()) / len(t)
    mean_b = sum(by.values()) / len(by)
    res = {"workload": wl.name, "heads": H, "positions": f"0..{W - 2}",
           "us_by_position": [round(t[n], 2) for n in pos],
           "gbps_by_position": [round(by[n] / (t[n] * 1e-6) / 1e9, 1) for n in pos],
           "us_mean": mean_us, "gbps_mean": mean_b / (mean_us * 1e-6) / 1e9,
           "read_ceiling_gbps": read_ceiling(int(mean_b), reps)}
    print(json.dumps(res), flush=True)
    return res


# ---------------------------------------------------------------- reductions
def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def counter_per_dispatch(path, kernel, counter):
    """Mean over dispatches of `kernel` (substring of the kernel name) of the
    counter's value (summed over the CSV's rows of one dispatch)."""
    per = {}
    for r in _rows(path):
        if kernel not in r.get("Kernel_Name", "") or r.get("Counter_Name") != counter:
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} rows for kernel {kernel!r} in {path}")
    vals = list(per.values())
    return sum(vals) / len(vals), len(vals)


def traffic(args):
    """HBM bytes per launch of `kernel` from FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each scaled by bytes-moved / counter of a plain copy."""
    copy_bytes = args.copy_mib * 2**20
    cf, _ = counter_per_dispatch(args.copy_fetch, args.copy_kernel, "FETCH_SIZE")
    cw, _ = counter_per_dispatch(args.copy_write, args.copy_kernel, "WRITE_SIZE")
    f_scale = copy_bytes / (cf * 1024.0)
    w_scale = copy_bytes / (cw * 1024.0)
    kf, nf = counter_per_dispatch(args.fetch, args.kernel, "FETCH_SIZE")
    kw, nw = counter_per_dispatch(args.write, args.kernel, "WRITE_SIZE")
    fetch_b = kf * 1024.0 * f_scale
    write_b = kw * 1024.0 * w_scale
    out = {
        "kernel": args.kernel,
        "kernel_sha": kernel_sha(args.kernel_src),
        "workload": args.workload,
        "dispatches": [nf, nw],
        "fetch_kib_raw": kf,
        "write_kib_raw": kw,
        "copy_mib": args.copy_mib,
        "copy_fetch_scale": f_scale,
        "copy_write_scale": w_scale,
        "fetch_bytes_per_launch": fetch_b,
        "write_bytes_per_launch": write_b,
        "bytes_per_launch": fetch_b + write_b,
    }
    with open(args.out, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def valu(args):
    """Per-launch VALU instructions, waves and matrix-core cycles of `kernel`."""
    want = {"SQ_INSTS_VALU": "insts_valu_per_launch", "SQ_WAVES": "waves_per_launch",
            "SQ_VALU_MFMA_BUSY_CYCLES": "mfma_busy_cycles_per_launch",
            "SQ_VALU_MFMA_COEXEC_CYCLES": "mfma_coexec_cycles_per_launch",
            "SQ_INSTS_MFMA": "insts_mfma_per_launch", "SQ_ACTIVE_INST_VALU": "active_inst_valu_per_launch"}
    out = {"kernel": args.kernel, "kernel_sha": kernel_sha(FOLD_SOURCES), "workload": args.workload}
    for path in args.csv:
        names = {r.get("Counter_Name") for r in _rows(path) if args.kernel in r.get("Kernel_Name", "")}
        for c in sorted(names & set(want)):
            if want[c] not in out:
                out[want[c]], n = counter_per_dispatch(path, args.kernel, c)
                out.setdefault("dispatches", n)
    for k in ("insts_valu_per_launch", "waves_per_launch", "mfma_busy_cycles_per_launch"):
        if k not in out:
            raise SystemExit(f"missing counter for {k}")
    out["insts_valu_per_wave"] = out["insts_valu_per_launch"] / out["waves_per_launch"]
    with open(args.out, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def stats(args):
    """Kernel-trace stats CSV -> a short table (name, calls, mean us, total ms)."""
    rows = _rows(args.csv)
    print(f"{'kernel':60s} {'calls':>6s} {'mean_us':>10s} {'total_ms':>10s} {'pct':>6s}")
    for r in rows:
        name = r["Name"][:60]
        print(f"{name:60s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
              f"{float(r['TotalDurationNs']) / 1e6:10.3f} {float(r['Percentage']):6.2f}")


def main(argv=None):
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--workload", default="b512")
    r.add_argument("--windows", type=int, default=2)
    r.add_argument("--fused", action="store_true")
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=1024)
    c.add_argument("--reps", type=int, default=4)
    cx = sub.add_parser("coexec")
    cx.add_argument("--agpr", action="store_true")
    cx.add_argument("--lds", type=int, default=40960)
    cx.add_argument("--reps", type=int, default=10)
    pt = sub.add_parser("pattern")
    pt.add_argument("--workload", default="b512")
    pt.add_argument("--reps", type=int, default=20)
    t = sub.add_parser("traffic")
    t.add_argument("--kernel", default="k_append<", help="substring of the kernel name")
    t.add_argument("--kernel-src", nargs="+", default=list(APPEND_SOURCES))
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-kernel", default="neg_kernel")
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--copy-mib", type=int, default=1024)
    t.add_argument("--workload", default="b512")
    t.add_argument("--out", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--csv", required=True)
    v = sub.add_parser("valu")
    v.add_argument("--kernel", default="k_append_fold")
    v.add_argument("--csv", action="append", required=True)
    v.add_argument("--workload", default="b512")
    v.add_argument("--out", required=True)
    a = p.parse_args(argv)
    if a.cmd == "run":
        run_layer(a.workload, a.windows, a.fused)
    elif a.cmd == "copy":
        run_copy(a.mib, a.reps)
    elif a.cmd == "coexec":
        run_coexec(a.agpr, a.lds, a.reps)
    elif a.cmd == "pattern":
        run_pattern(a.workload, a.reps)
    elif a.cmd == "traffic":
        traffic(a)
    elif a.cmd == "valu":
        valu(a)
    else:
        stats(a)


if __name__ == "__main__":
    main()
