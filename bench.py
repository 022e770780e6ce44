"""Benchmark of the fused EM iteration on one MI355X.

A step is one EM iteration (gmm_fit_step: precision prologue, fused E-step
with statistics, deterministic reduction, M-step) over the whole synthetic
workload, with the rows already resident in device memory.  The default
workload is the diagonal-covariance one (N = 1,000,000 rows, D = 64, K = 256,
float32); the others are available with --workload.

Prints ONE JSON line (rank 0): value = points*components per second
(B*N*K / time per iteration), plus the roofline of the fused E-step kernel
(timed with HIP events that the library records around that kernel on the
stream it runs on) and the float64 CPU oracle timed on the host cores on a
bounded sample of the same workload.
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
    pass C (4 x 2D), statistics in two magnitude classes over D features plus
    the 16-feature block that carries 1 and |x|^2 (2 x 2 (D + 16))."""
    return 4 * D + 4, 8 * D + 4 * (D + 16)


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


def cpu_baseline(wl, budget_s=20.0, max_steps=4, target_macs=2e10):
    """The float64 oracle's EM iteration on the host cores, on the first rows of
    the workload (all of them when one iteration stays near target_macs
    multiply-adds), reported per point*component."""
    import oracle
    nthreads = os.cpu_count() or 1
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
            "kind": "oracle",
            "sample": f"{len(times)} float64 EM iterations of {what} {wl.name} workload "
                      f"(B={wl.B}, N={wl.N}, D={wl.D}, K={wl.K}) from theta_0, median "
                      f"{t:.2f} s/iteration"}


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
        res["cpu_baseline"] = {"value": q * M / t, "unit": "pairs/s", "cores": 1, "kind": "oracle",
                               "sample": f"oracle.kde_score (numpy float64, direct differences) on the first {q} "
                                         f"queries against all {M} references, {t:.1f} s"}
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="diag_large",
                    choices=["diag_large", "spherical_small", "diag_batched", "full_large", "ivf_bf16", "kde"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--calib-copy", type=int, default=0,
                    help="also run a plain device copy of this many MiB (traffic counter calibration)")
    args = ap.parse_args()
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
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        g.gmm_fit_step(X, w, mu, cv, wl.cov, reg_covar=wl.eps, mean_loglik=mll, ws=ws, events=evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_s = (t1 - t0) / args.steps
    k_ms = float(np.mean([a_.elapsed_time(b_) for a_, b_ in evs]))

    pairs = wl.B * wl.N * wl.K
    if wl.xdtype == "bf16":
        alg, executed = largek_roofline(wl.D)
        flops = pairs * alg
        peak = PEAK_BF16_MFMA
        kernel = "large-K E-step (prologue + passes A, B, C)"
        peak_note = (f"bf16 MFMA dense peak; {alg} algorithmic flop/pair (2D logits + 2D statistics); "
                     f"{executed} flop/pair executed (two-term weights, logits recomputed in pass C, "
                     f"statistics in two magnitude classes)")
        dtype = "bf16"
    else:
        f32f, f64f = contraction_split(wl.cov, wl.D)
        flops = pairs * (f32f + f64f)
        peak = (f32f + f64f) / (f32f / PEAK_FP32_MFMA + f64f / PEAK_FP64_MFMA)
        kernel = "fused E-step + statistics"
        peak_note = (f"float32 MFMA logits ({f32f} flop/pair at {PEAK_FP32_MFMA} TF) + float64 MFMA "
                     f"statistics ({f64f} flop/pair at {PEAK_FP64_MFMA} TF), time-weighted")
        dtype = "f32"
    achieved = flops / (k_ms * 1e-3) / 1e12
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
            "traffic": measured_traffic(wl.name, "gmm_largek.hip" if wl.xdtype == "bf16" else "gmm_estep.hip"),
            "traffic_unit": "bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "kernel": kernel,
            "kernel_ms": k_ms,
            "flops_per_launch": flops,
            "peak_note": peak_note,
        },
        "mean_loglik_last": float(mll.mean().item()),
    }
    if wl.topm is not None:
        # soft multi-assignment under the fitted model: one pass, timed apart
        m, thr = wl.topm
        idx = torch.empty((wl.B, wl.N, m), dtype=torch.int32, device=dev)
        resp = torch.empty((wl.B, wl.N, m), dtype=torch.float32, device=dev)
        cnt = torch.empty((wl.B, wl.N), dtype=torch.int32, device=dev)
        tws = torch.empty(g.gmm_workspace_bytes(X, wl.K, wl.cov, op=g.OP_TOPM, m=m), dtype=torch.uint8,
                          device=dev)
        g.gmm_predict_proba_topm(X, w, mu, cv, wl.cov, m, thr, idx, resp, cnt, ws=tws)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g.gmm_predict_proba_topm(X, w, mu, cv, wl.cov, m, thr, idx, resp, cnt, ws=tws)
        torch.cuda.synchronize()
        t_topm = time.perf_counter() - t0
        res["topm"] = {"m": m, "threshold": thr, "ms": t_topm * 1e3, "rows_per_s": wl.B * wl.N / t_topm,
                       "mean_kept": float(cnt.float().mean().item())}
        # the IVF posting lists of that assignment (CSR per component), timed apart
        off = torch.empty((wl.B, wl.K + 1), dtype=torch.int64, device=dev)
        rows = torch.empty((wl.B, wl.N * m), dtype=torch.int32, device=dev)
        lresp = torch.empty((wl.B, wl.N * m), dtype=torch.float32, device=dev)
        lws = torch.empty(max(256, g.gmm_ivf_workspace_bytes(wl.B, wl.N, m, wl.K)), dtype=torch.uint8, device=dev)
        g.gmm_ivf_lists(idx, wl.K, resp=resp, offsets=off, rows=rows, list_resp=lresp, ws=lws)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
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
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
