"""Benchmark of the fused EM iteration on one MI355X.

A step is one EM iteration (gmm_fit_step: precision prologue, E-step with
statistics, deterministic reduction, M-step) over the whole synthetic
workload, with the rows already resident in device memory.  The default
workload is the largest configuration that fits one GPU: the IVF coarse
quantizer (spherical GMM, N = 10,000,000 bf16 rows, D = 128, K = 4096); the
others are available with --workload.

Prints ONE JSON line (rank 0): value = points*components per second
(B*N*K / time per iteration), plus the roofline of the E-step (timed with HIP
events that the library records around it on the stream it runs on) against
the dense MFMA peak of the type its contractions run in (bf16 for bf16 rows,
float32 otherwise), and the float64 CPU oracle timed on the host cores on a
bounded sample of the same workload.

The timed loop is bracketed by two short spin kernels (torch.cuda._sleep),
outside the timed region, so that a kernel trace of the same command can be
cut to the timed dispatches:  python bench.py --summarize DIR  prints the
per-kernel summary of the rocprofv3 kernel trace under DIR between those
markers (and, with --counters, the per-kernel sums of the counters of a
rocprofv3 --pmc run, calibrated by the --calib-copy copy kernel).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("EM iterations/sec and N·K points·components/s per iteration; "
          "% MFMA or HBM roofline")

# MI355X published dense peaks (TFLOP/s)
PEAK_FP32_MFMA = 157.3
PEAK_FP64_MFMA = 78.6
PEAK_BF16_MFMA = 2500.0


def flops_per_pair(cov, D):
    """Algorithmic flops per (point, component) of the two contractions
    (2 per multiply-add) plus the N_k sum: logits over F features, statistics
    over the same F features."""
    if cov == "spherical":
        f = D              # x . (lambda mu); |x|^2 term on the VALU
        return 4 * f + 4   # + |x|^2 coefficient, N_k, sum r|x|^2
    if cov == "diag":
        return 8 * D + 2
    q = D * (D + 1) // 2
    return 4 * (D + q) + 2


def largek_roofline(D):
    """(algorithmic flops, executed flops) per pair of the bf16 large-K E-step.
    Algorithmic: logits 2D and statistics 2D, plus N_k and sum r|x|^2.
    Executed: logits with the hi and lo weight terms in pass A and again in
    pass C (4 x 2D), pass A's 16-feature step for c + a |x|^2 (2 x 16),
    statistics in two magnitude classes over D features plus the 16-feature
    block that carries 1 and |x|^2 (2 x 2 (D + 16))."""
    return 4 * D + 4, 8 * D + 2 * 16 + 4 * (D + 16)


def contraction_split(cov, D):
    """(float32 flops, float64 flops) per pair: logits run on the float32 MFMA,
    statistics on the float64 MFMA."""
    total = flops_per_pair(cov, D)
    half = total // 2
    return half, total - half


def measured_traffic(workload, source):
    """HBM bytes per launch of the E-step from the committed counter summary,
    if it was taken on this workload with the current kernel source."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", f"estep_{workload}_traffic.md")
    src = os.path.join(ROOT, "soft_clustering_em_amd", "csrc", source)
    if not os.path.exists(path):
        return None
    m = re.search(r"<!-- machine-readable: (\{.*\}) -->", open(path).read())
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec["kernel_sha256"] != hashlib.sha256(open(src, "rb").read()).hexdigest():
        return None
    return rec["fetch_bytes"] + rec["write_bytes"]


def host_threads():
    """Threads the oracle may use: the cores this process may run on, capped by
    OMP_NUM_THREADS when that is set."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    cap = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    return max(1, min(n, cap) if cap > 0 else n)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, budget_s=20.0, max_steps=4, target_macs=2e10):
    """The float64 oracle's EM iteration on the host cores, on the first rows of
    the workload (all of them when one iteration stays near target_macs
    multiply-adds), reported per point*component."""
    import oracle
    nthreads = host_threads()
    per_pair = wl.D * (wl.D + 1) if wl.cov in ("full", "tied") else wl.D
    rows = int(min(wl.N, max(1024, target_macs // (wl.B * wl.K * per_pair))))
    Xs = wl.X[:, :rows]
    X = Xs if wl.xdtype == "f32" else (Xs, "bf16")
    w, mu, cv = (a.astype(np.float64) for a in (wl.w0, wl.mu0, wl.cv0))
    times = []
    t_start = time.perf_counter()
    for _ in range(max_steps):
        t0 = time.perf_counter()
        out = oracle.fit_step(wl.cov, X, w, mu, cv, eps=wl.eps, nthreads=nthreads)
        times.append(time.perf_counter() - t0)
        w, mu, cv = out["w"], out["mu"], out["cv"]
        if time.perf_counter() - t_start > budget_s:
            break
    t = float(np.median(times))
    what = "the full" if rows == wl.N else f"the first {rows} rows of the"
    return {"value": wl.B * rows * wl.K / t, "unit": "points*components/s", "cores": nthreads,
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{len(times)} float64 EM iterations of {what} {wl.name} workload "
                      f"(B={wl.B}, N={wl.N}, D={wl.D}, K={wl.K}) from theta_0, median "
                      f"{t:.2f} s/iteration"}


def _read_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find(root, suffix):
    out = []
    for d, _, files in os.walk(root):
        out += [os.path.join(d, f) for f in files if f.endswith(suffix)]
    return sorted(out)


def _window(rows):
    """(first, last) dispatch ids strictly between the first two spin-kernel
    markers, or None when the trace has fewer than two."""
    marks = sorted({int(r["Dispatch_Id"]) for r in rows if "spin" in r["Kernel_Name"].lower()})
    if len(marks) < 2:
        return None
    # the two markers of the timed loop are consecutive spin dispatches
    return marks[0], marks[1]


def _short(name, n=90):
    name = name.replace("gmm::(anonymous namespace)::", "gmm::")
    return name if len(name) <= n else name[:n] + "..."


def summarize(root, counters, calib_mib):
    """Markdown summary of rocprofv3 output under root.  Trace: per-kernel
    calls and durations of the dispatches between the timed-loop markers, then
    of those after them.  Counters: per kernel in the timed window, the
    counters' mean per dispatch; FETCH_SIZE / WRITE_SIZE also scaled by what
    they read on the calibration copy of calib_mib MiB (the copy kernel before
    the window with the largest counts: smaller copies of the model state may
    follow it)."""
    if not counters:
        files = _find(root, "kernel_trace.csv")
        if not files:
            sys.exit(f"no kernel_trace.csv under {root}")
        rows = [r for f in files for r in _read_csv(f)]
        win = _window(rows)

        def table(sel, title):
            agg = {}
            for r in sel:
                d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
                agg.setdefault(r["Kernel_Name"], []).append(d)
            tot = sum(sum(v) for v in agg.values())
            print(f"\n{title}\n")
            print("| kernel | calls | total (us) | average (us) | min (us) | max (us) | share |")
            print("|---|---|---|---|---|---|---|")
            for k, v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
                print(f"| `{_short(k)}` | {len(v)} | {sum(v):.1f} | {sum(v) / len(v):.1f} | {min(v):.1f} | "
                      f"{max(v):.1f} | {100 * sum(v) / tot:.1f}% |")
            print(f"\nSum of kernel durations: {tot:.1f} us.")

        if win is None:
            table(rows, "All dispatches (no timed-loop markers in this trace):")
            return
        lo, hi = win
        timed = [r for r in rows if lo < int(r["Dispatch_Id"]) < hi]
        after = [r for r in rows if int(r["Dispatch_Id"]) > hi and "spin" not in r["Kernel_Name"].lower()]
        table(timed, f"Timed loop (dispatches {lo + 1}..{hi - 1}, between the markers):")
        if after:
            table(after, "After the timed loop (top-m pass, posting lists, k-means step where the workload has them):")
        return
    files = _find(root, "counter_collection.csv")
    if not files:
        sys.exit(f"no counter_collection.csv under {root}")
    rows = [r for f in files for r in _read_csv(f)]
    win = _window(rows)
    per = {}
    for r in rows:
        per.setdefault((int(r["Dispatch_Id"]), r["Kernel_Name"]), {})[r["Counter_Name"]] = float(r["Counter_Value"])
    scale = {}
    if calib_mib and win is not None:
        copies = [(d, c) for (d, k), c in per.items() if "copy" in k.lower() and d < win[0]]
        if copies:
            kib = calib_mib * 1024.0
            c = max(copies, key=lambda dc: max(dc[1].values()))[1]
            for name in ("FETCH_SIZE", "WRITE_SIZE"):
                if c.get(name):
                    scale[name] = kib / c[name]
            print(f"Calibration copy of {calib_mib} MiB ({kib:.0f} KiB read and written): "
                  + ", ".join(f"{n} reads {c[n]:.1f} KiB (factor {scale[n]:.4f})" for n in scale))
    agg = {}
    for (d, k), c in per.items():
        if win is not None and not (win[0] < d < win[1]):
            continue
        a = agg.setdefault(k, {"n": 0})
        a["n"] += 1
        for n, v in c.items():
            a[n] = a.get(n, 0.0) + v
    names = sorted({n for a in agg.values() for n in a if n != "n"})
    print("\n| kernel | dispatches | " + " | ".join(f"{n} (mean)" for n in names) + " |")
    print("|---|---|" + "---|" * len(names))
    for k, a in sorted(agg.items(), key=lambda kv: kv[0]):
        print(f"| `{_short(k)}` | {a['n']} | " + " | ".join(f"{a.get(n, 0.0) / a['n']:.4g}" for n in names) + " |")
    for n in scale:
        tot = sum(a.get(n, 0.0) for a in agg.values())
        print(f"\n{n}: {tot:.1f} KiB over the window, {tot * scale[n] * 1024:.4g} bytes scaled")


def run_kde(args, torch, g, synth):
    """Gaussian kernel density estimate: 1,000,000 query rows against 65,536
    reference rows, D = 64, float32, bandwidth by Scott's rule.  A step is one
    gmm_kde_score call (reference centring, then the streaming kernel)."""
    Y, X, h = synth.kde_inputs()
    N, D = Y.shape
    M = X.shape[0]
    Yd, Xd = torch.from_numpy(Y).cuda(), torch.from_numpy(X).cuda()
    out = torch.empty(N, dtype=torch.float32, device="cuda")
    ws = torch.empty(g.gmm_kde_workspace_bytes(Yd, M), dtype=torch.uint8, device="cuda")
    for _ in range(args.warmup):
        g.gmm_kde_score(Yd, Xd, h, out=out, ws=ws)
    torch.cuda.synchronize()
    # the library launches on torch's current stream, where these events are recorded
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        g.gmm_kde_score(Yd, Xd, h, out=out, ws=ws)
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    ms = e0.elapsed_time(e1) / args.steps
    pairs = N * M
    flops = 2 * D * pairs  # the cross-term contraction y . x
    achieved = flops / (ms * 1e-3) / 1e12
    res = {
        "metric": "kernel density: query*reference pairs/s; % of the float32 MFMA peak",
        "value": pairs / wall,
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "kde", "N": N, "M": M, "D": D, "bandwidth": h},
        "roofline": {
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_FP32_MFMA,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_FP32_MFMA,
            "traffic": None,
            "kernel": "kernel density call (centring kernels + streaming kernel)",
            "kernel_ms": ms,
            "flops_per_launch": flops,
            "peak_note": "2 D flops per pair (the cross terms on v_mfma_f32_16x16x4_f32)",
        },
        "mean_logdens": float(out.double().mean().item()),
    }
    if not args.no_cpu:
        import oracle
        q = 2000
        t0 = time.perf_counter()
        oracle.kde_score(Y[:q], X, h)
        t = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": q * M / t, "unit": "pairs/s", "cores": 1, "cpu_model": cpu_model(),
                               "kind": "oracle",
                               "sample": f"oracle.kde_score (numpy float64, direct differences) on the first {q} "
                                         f"queries against all {M} references, {t:.1f} s"}
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="ivf_bf16",
                    choices=["diag_large", "spherical_small", "diag_batched", "full_large", "ivf_bf16", "kde",
                             "diag_blocked"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--streamed", type=int, default=0, metavar="CHUNK",
                    help="also time gmm_fit_step_streamed from pinned host rows in chunks of CHUNK rows "
                         "(the PCIe-inclusive rate; reported under 'streamed', never as the value)")
    ap.add_argument("--no-topm", action="store_true",
                    help="skip the top-m / posting-list / k-means measurements after the fit (counter runs)")
    ap.add_argument("--calib-copy", type=int, default=0,
                    help="also run a plain device copy of this many MiB (traffic counter calibration)")
    ap.add_argument("--summarize", metavar="DIR",
                    help="summarise the rocprofv3 output under DIR (no GPU work)")
    ap.add_argument("--counters", action="store_true", help="with --summarize: counter (--pmc) output")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize, args.counters, args.calib_copy)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)

    import torch
    import soft_clustering_em_amd as g
    from soft_clustering_em_amd import synth

    dev = "cuda"
    torch.cuda.init()
    if args.workload == "kde":
        run_kde(args, torch, g, synth)
        return
    wl = synth.WORKLOADS[args.workload]()
    if wl.xdtype == "bf16":
        X = torch.from_numpy(wl.X.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        X = torch.from_numpy(wl.X).to(dev)
    w = torch.from_numpy(wl.w0.copy()).to(dev)
    mu = torch.from_numpy(wl.mu0.copy()).to(dev)
    cv = torch.from_numpy(wl.cv0.copy()).to(dev)
    mll = torch.zeros(wl.B, dtype=torch.float64, device=dev)
    ws = torch.empty(g.gmm_workspace_bytes(X, wl.K, wl.cov), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    if args.calib_copy:
        n = args.calib_copy * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    for _ in range(args.warmup):
        g.gmm_fit_step(X, w, mu, cv, wl.cov, reg_covar=wl.eps, mean_loglik=mll, ws=ws)
    torch.cuda.synchronize()

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a_, b_ in evs:  # materialise the event handles before handing them to the library
        a_.record(stream)
        b_.record(stream)
    theta_in = tuple(t_.clone() for t_ in (w, mu, cv))  # the state the timed loop starts from
    torch.cuda._sleep(1000)  # trace marker: the timed dispatches follow
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        g.gmm_fit_step(X, w, mu, cv, wl.cov, reg_covar=wl.eps, mean_loglik=mll, ws=ws, events=evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    torch.cuda._sleep(1000)  # trace marker: the timed dispatches ended
    step_s = (t1 - t0) / args.steps
    k_ms = float(np.mean([a_.elapsed_time(b_) for a_, b_ in evs]))

    pairs = wl.B * wl.N * wl.K
    extra = {}
    if wl.xdtype == "bf16":
        alg, executed = largek_roofline(wl.D)
        flops = pairs * alg
        peak = PEAK_BF16_MFMA
        kernel = "large-K E-step (prologue + passes A, B, C over every row chunk)"
        peak_note = (f"bf16 MFMA dense peak; {alg} algorithmic flop/pair (2D logits + 2D statistics + N_k and "
                     f"|x|^2 terms)")
        extra = {"executed_flops_per_launch": pairs * executed,
                 "executed_frac": pairs * executed / (k_ms * 1e-3) / 1e12 / peak,
                 "executed_note": (f"{executed} flop/pair executed: two-term weights, logits again in pass C, c + a|x|^2 step in pass A, "
                                   f"statistics in two magnitude classes")}
        dtype = "bf16"
    else:
        f32f, f64f = contraction_split(wl.cov, wl.D)
        flops = pairs * (f32f + f64f)
        peak = PEAK_FP32_MFMA
        blend = (f32f + f64f) / (f32f / PEAK_FP32_MFMA + f64f / PEAK_FP64_MFMA)
        kernel = ("fused E-step + statistics" if wl.K <= 256 else
                  "fused E-step in blocks of components (max/sum pass, row combine, statistics pass per row chunk)")
        peak_note = (f"float32 MFMA dense peak; {f32f + f64f} algorithmic flop/pair (logits and statistics "
                     f"contractions)")
        extra = {"frac_vs_fp32_fp64_blend": flops / (k_ms * 1e-3) / 1e12 / blend,
                 "blend_note": (f"secondary: the statistics half runs on the float64 MFMA; blended peak "
                                f"{blend:.1f} TF for {f32f} float32 + {f64f} float64 flop/pair")}
        dtype = "f32"
    achieved = flops / (k_ms * 1e-3) / 1e12
    tr = measured_traffic(wl.name, "gmm_largek.hip" if wl.xdtype == "bf16" else "gmm_estep.hip")
    res = {
        "metric": METRIC,
        "value": pairs / step_s,
        "unit": "points*components/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "iters_per_sec": 1.0 / step_s,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "cov": wl.cov, "B": wl.B, "N": wl.N, "D": wl.D, "K": wl.K,
                   "iters_per_fit": wl.iters},
        "roofline": {
            "bound": "mfma",
            "achieved": achieved,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": achieved / peak,
            "traffic": tr,
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "traffic_source": (f"profiles/estep_{wl.name}_traffic.md (taken with the current kernel source)"
                               if tr is not None else "none for the current kernel source"),
            "kernel": kernel,
            "kernel_ms": k_ms,
            "flops_per_launch": flops,
            "peak_note": peak_note,
            **extra,
        },
        "mean_loglik_last": float(mll.mean().item()),
    }
    # the same iterations from the same state through one gmm_fit call (after
    # the first iteration, each prologue is formed by the previous M-step: one
    # launch fewer per iteration on the fused path), timed apart
    mlls = torch.zeros((args.steps, wl.B), dtype=torch.float64, device=dev)
    for t_, s_ in zip((w, mu, cv), theta_in):
        t_.copy_(s_)
    g.gmm_fit(X, w, mu, cv, wl.cov, 1, reg_covar=wl.eps, mean_loglik=mlls, ws=ws)
    for t_, s_ in zip((w, mu, cv), theta_in):
        t_.copy_(s_)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.gmm_fit(X, w, mu, cv, wl.cov, args.steps, reg_covar=wl.eps, mean_loglik=mlls, ws=ws)
    torch.cuda.synchronize()
    t_fit = (time.perf_counter() - t0) / args.steps
    res["fit_call"] = {"n_iter": args.steps, "ms_per_step": t_fit * 1e3, "points_components_per_s": pairs / t_fit,
                       "note": "gmm_fit: the iterations in one call, each next prologue formed by the M-step"}
    if wl.topm is not None and not args.no_topm:
        # soft multi-assignment under the fitted model: one pass, timed apart
        m, thr = wl.topm
        idx = torch.empty((wl.B, wl.N, m), dtype=torch.int32, device=dev)
        resp = torch.empty((wl.B, wl.N, m), dtype=torch.float32, device=dev)
        cnt = torch.empty((wl.B, wl.N), dtype=torch.int32, device=dev)
        tws = torch.empty(g.gmm_workspace_bytes(X, wl.K, wl.cov, op=g.OP_TOPM, m=m), dtype=torch.uint8,
                          device=dev)
        g.gmm_predict_proba_topm(X, w, mu, cv, wl.cov, m, thr, idx, resp, cnt, ws=tws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.gmm_predict_proba_topm(X, w, mu, cv, wl.cov, m, thr, idx, resp, cnt, ws=tws)
        e1.record()
        torch.cuda.synchronize()
        t_topm = e0.elapsed_time(e1) * 1e-3
        res["topm"] = {"m": m, "threshold": thr, "ms": t_topm * 1e3, "rows_per_s": wl.B * wl.N / t_topm,
                       "mean_kept": float(cnt.float().mean().item())}
        # the IVF posting lists of that assignment (CSR per component), timed apart
        off = torch.empty((wl.B, wl.K + 1), dtype=torch.int64, device=dev)
        rows = torch.empty((wl.B, wl.N * m), dtype=torch.int32, device=dev)
        lresp = torch.empty((wl.B, wl.N * m), dtype=torch.float32, device=dev)
        lws = torch.empty(max(256, g.gmm_ivf_workspace_bytes(wl.B, wl.N, m, wl.K)), dtype=torch.uint8, device=dev)
        g.gmm_ivf_lists(idx, wl.K, resp=resp, offsets=off, rows=rows, list_resp=lresp, ws=lws)
        reps = 5
        e0.record()
        for _ in range(reps):
            g.gmm_ivf_lists(idx, wl.K, resp=resp, offsets=off, rows=rows, list_resp=lresp, ws=lws)
        e1.record()
        torch.cuda.synchronize()
        t_lists = e0.elapsed_time(e1) / reps
        entries = int(off[:, wl.K].sum().item())
        # bytes each build moves at the least: idx read twice (count and place),
        # resp read once, rows and responsibilities written once per entry
        lbytes = wl.B * wl.N * m * 4 * 3 + entries * 8
        res["topm"]["ivf_lists"] = {"ms": t_lists, "entries": entries, "entries_per_s": entries / (t_lists * 1e-3),
                                    "algorithmic_bytes": lbytes, "achieved_GBs": lbytes / (t_lists * 1e-3) / 1e9}
        # the hard-assignment baseline: Lloyd steps from the fitted means
        # (nearest centroid, posting lists of the labels, cluster means)
        if wl.B == 1:
            C = mu.clone().contiguous()
            kws = torch.empty(g.gmm_kmeans_workspace_bytes(X, wl.K), dtype=torch.uint8, device=dev)
            lab = torch.empty((wl.B, wl.N), dtype=torch.int32, device=dev)
            kcnt = torch.empty((wl.B, wl.K), dtype=torch.int64, device=dev)
            kin = torch.empty((wl.B,), dtype=torch.float64, device=dev)
            g.gmm_kmeans_step(X, C, lab, kcnt, kin, ws=kws)
            reps = 3
            e0.record()
            for _ in range(reps):
                g.gmm_kmeans_step(X, C, lab, kcnt, kin, ws=kws)
            e1.record()
            torch.cuda.synchronize()
            t_km = e0.elapsed_time(e1) / reps
            res["topm"]["kmeans_step"] = {"ms": t_km, "points_components_per_s": wl.N * wl.K / (t_km * 1e-3),
                                          "inertia_last": float(kin[0].item())}
    if args.streamed:
        # the same EM iteration with the rows in pinned host memory, copied in
        # chunks on a second stream while the previous chunk's E-step runs
        Xh = torch.empty(X.shape, dtype=X.dtype, pin_memory=True)
        Xh.copy_(X.cpu())
        sws = torch.empty(g.gmm_fit_step_streamed_workspace_bytes(Xh, wl.K, wl.cov, args.streamed), dtype=torch.uint8,
                          device=dev)
        copy = torch.cuda.Stream()
        for t_, a_ in ((w, wl.w0), (mu, wl.mu0), (cv, wl.cv0)):
            t_.copy_(torch.from_numpy(a_))
        g.gmm_fit_step_streamed(Xh, w, mu, cv, wl.cov, args.streamed, reg_covar=wl.eps, ws=sws, copy_stream=copy)
        torch.cuda.synchronize()
        reps = 3
        t0 = time.perf_counter()
        for _ in range(reps):
            g.gmm_fit_step_streamed(Xh, w, mu, cv, wl.cov, args.streamed, reg_covar=wl.eps, ws=sws, copy_stream=copy)
        torch.cuda.synchronize()
        t_s = (time.perf_counter() - t0) / reps
        hbytes = Xh.numel() * Xh.element_size()
        res["streamed"] = {"chunk_rows": args.streamed, "ms_per_step": t_s * 1e3, "points_components_per_s": pairs / t_s,
                           "host_GBs": hbytes / t_s / 1e9, "device_workspace_bytes": sws.numel(),
                           "rows_bytes": hbytes}
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
