"""Shared helpers of the GPU parity tests: oracle trajectories and the
tolerance metrics used to compare one EM step of the HIP library with one
step of the float64 oracle from identical float32 parameters.

Metrics (relative unless stated):
  means      per component |mu_g - mu_o| / max(|mu_o|, sqrt(tr Sigma_o))
  variances  element-wise (spherical, diag); Frobenius per matrix (full, tied)
  weights    where pi_o >= 1e-6; absolute 1e-10 below
  mean LL    relative
Components whose oracle N_k < 1 are excluded from the mean / variance checks.
Tolerance: 1e-4 for float32 rows, 2e-2 for bf16/f16 rows.
"""
from __future__ import annotations

import numpy as np

import oracle

TOL_F32 = 1e-4
TOL_LOWP = 2e-2


def to_np(t):
    return t.detach().to("cpu").numpy().astype(np.float64)


def trace_cov(cov, cv, B, K, D):
    if cov == "spherical":
        return D * cv.reshape(B, K)
    if cov == "diag":
        return cv.reshape(B, K, D).sum(-1)
    if cov == "full":
        return np.trace(cv.reshape(B, K, D, D), axis1=-2, axis2=-1)
    return np.repeat(np.trace(cv.reshape(B, D, D), axis1=-2, axis2=-1)[:, None], K, 1)


def param_errors(cov, B, K, D, got, ref, nk_ref):
    """got/ref: (w, mu, cv) float64 arrays.  Returns dict of max errors."""
    wg, mg, cg = (np.asarray(a, np.float64) for a in got)
    wo, mo, co = (np.asarray(a, np.float64) for a in ref)
    wg, wo = wg.reshape(B, K), wo.reshape(B, K)
    mg, mo = mg.reshape(B, K, D), mo.reshape(B, K, D)
    live = nk_ref.reshape(B, K) >= 1.0
    scale = np.maximum(np.linalg.norm(mo, axis=-1), np.sqrt(np.abs(trace_cov(cov, co, B, K, D))))
    e_mu = np.linalg.norm(mg - mo, axis=-1) / scale
    big = wo >= 1e-6
    e_w = np.where(big, np.abs(wg - wo) / np.where(big, wo, 1.0), 0.0)
    e_w_small = np.where(~big, np.abs(wg - wo), 0.0)
    if cov in ("spherical", "diag"):
        cgs = cg.reshape(B, K, -1)
        cos = co.reshape(B, K, -1)
        e_cv = (np.abs(cgs - cos) / np.abs(cos)).max(-1)
        e_cv = np.where(live, e_cv, 0.0)
    elif cov == "full":
        cgs, cos = cg.reshape(B, K, D, D), co.reshape(B, K, D, D)
        e_cv = np.linalg.norm(cgs - cos, axis=(-2, -1)) / np.linalg.norm(cos, axis=(-2, -1))
        e_cv = np.where(live, e_cv, 0.0)
    else:
        cgs, cos = cg.reshape(B, D, D), co.reshape(B, D, D)
        e_cv = np.linalg.norm(cgs - cos, axis=(-2, -1)) / np.linalg.norm(cos, axis=(-2, -1))
    return dict(mu=float(np.where(live, e_mu, 0.0).max()), cv=float(np.max(e_cv)),
                w=float(e_w.max()), w_abs_small=float(e_w_small.max()), live=int(live.sum()))


def oracle_trajectory(wl, steps, nthreads=0):
    """theta_t as float32 arrays for t = 0..steps, each obtained by one float64
    oracle step from the float32 rounding of the previous one; also the oracle
    step outputs (float64) for t = 0..steps-1."""
    cov = wl.cov
    th = (wl.w0.astype(np.float32), wl.mu0.astype(np.float32), wl.cv0.astype(np.float32))
    thetas, outs = [th], []
    X = wl.X if wl.xdtype == "f32" else (wl.X, "bf16")
    for _ in range(steps):
        w, mu, cv = (a.astype(np.float64) for a in th)
        out = oracle.fit_step(cov, X, w, mu, cv, eps=wl.eps, nthreads=nthreads)
        outs.append(out)
        th = (out["w"].astype(np.float32).reshape(wl.w0.shape),
              out["mu"].astype(np.float32).reshape(wl.mu0.shape),
              out["cv"].astype(np.float32).reshape(wl.cv0.shape))
        thetas.append(th)
    return thetas, outs
