"""Float64 CPU oracle for one EM iteration of a Gaussian mixture model.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``; the product path never imports it.
The arithmetic lives in ``gmm_oracle.c`` (plain C, float64, OpenMP over rows);
this module builds it with gcc and marshals numpy arrays through ctypes.

Sources it follows: "Flash-GMM: A Memory-Efficient Kernel for Scalable Soft
Clustering", Section 2 (E-step score, log-sum-exp responsibilities, M-step
eqs. 1-3) and Section 4 / Conclusion (multi-assignment by a threshold on the
final responsibilities), and its closing discussion (Fisher vectors, kernel
density estimation); "ML0094 GMM vs K-Means", Mathematical Formulation
(responsibility-weighted covariance) and its k-means limit (kmeans_step); GMMXX README, Covariance Coverage (the
four covariance types and their shapes).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

COV = {"spherical": 0, "diag": 1, "tied": 2, "full": 3}
XTYPE = {"f64": 0, "f32": 1, "bf16": 2, "f16": 3}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gmm_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile gmm_oracle.c into liboracle.so with gcc (no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.oracle_estep.argtypes = [i32, i32, i64, i32, i32, P, i32, P, P, P, P, P, P, P, P, i32]
        lib.oracle_mstep.argtypes = [i32, i32, i64, i32, i32, P, P, P, P, P, P, f64, P, P, P, P]
        lib.oracle_mstep_twopass.argtypes = [i32, i64, i32, i32, P, i32, P, P, P, f64, P, P, P]
        lib.oracle_responsibilities.argtypes = [i32, i64, i32, i32, P, i32, P, P, P, P, P, P]
        lib.oracle_topm.argtypes = [i32, i64, i32, i32, P, i32, P, P, P, i32, f64, P, P, P, P, P, i32]
        lib.oracle_kmeans_step.argtypes = [i64, i32, i32, P, i32, P, P, P, P, P, P, i32]
        lib.oracle_decode.argtypes = [i32, i64, P, P]
        lib.oracle_decode.restype = ctypes.c_int
        for f in (lib.oracle_estep, lib.oracle_mstep, lib.oracle_mstep_twopass,
                  lib.oracle_responsibilities, lib.oracle_topm, lib.oracle_kmeans_step):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def _x_and_type(X):
    """X is float64/float32 ndarray, or a (uint16 ndarray, 'bf16'|'f16') pair."""
    if isinstance(X, tuple):
        arr, kind = X
        arr = np.ascontiguousarray(arr, dtype=np.uint16)
        return arr, XTYPE[kind]
    arr = np.ascontiguousarray(X)
    if arr.dtype == np.float64:
        return arr, XTYPE["f64"]
    if arr.dtype == np.float32:
        return arr, XTYPE["f32"]
    raise TypeError("oracle input must be float32/float64 or (uint16, 'bf16'|'f16')")


def decode_rows(X) -> np.ndarray:
    """The rows as float64, decoded exactly: float32/float64 arrays as they
    are; (uint16 bits, 'bf16') as bfloat16 (the upper half of a float32);
    (uint16 bits, 'f16') as IEEE binary16."""
    if isinstance(X, tuple):
        arr, kind = X
        bits = np.ascontiguousarray(arr, dtype=np.uint16)
        if kind == "bf16":
            return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
        if kind == "f16":
            return bits.view(np.float16).astype(np.float64)
        raise TypeError("unknown 16-bit row type %r" % (kind,))
    return np.asarray(X, dtype=np.float64)


def c_decode(X) -> np.ndarray:
    """The rows as the C oracle decodes them (float64, flattened)."""
    Xa, xt = _x_and_type(X)
    out = np.zeros(Xa.size)
    if _load().oracle_decode(xt, Xa.size, _ptr(Xa), _ptr(out)):
        raise ValueError("oracle_decode rejected its arguments")
    return out


def cov_len(cov: str, D: int, K: int) -> int:
    return {"spherical": K, "diag": K * D, "tied": D * D, "full": K * D * D}[cov]


def _params(w, mu, cv, B, K, D, cov):
    w = np.ascontiguousarray(w, dtype=np.float64).reshape(B, K)
    mu = np.ascontiguousarray(mu, dtype=np.float64).reshape(B, K, D)
    cv = np.ascontiguousarray(cv, dtype=np.float64).reshape(B, cov_len(cov, D, K))
    return w, mu, cv


def estep(cov, X, w, mu, cv, nthreads=0):
    """Sufficient statistics of one E-step.  X shape (B,N,D) or (N,D).

    Returns dict(nk (B,K), sx (B,K,D), sxx (B,len), ll (B) = sum_i log p(x_i),
    flags (B,K)).  sxx is centred at the means `mu` that entered the step.
    """
    Xa, xt = _x_and_type(X)
    single = Xa.ndim == 2
    if single:
        Xa = Xa[None]
    B, N, D = Xa.shape
    K = np.asarray(w).reshape(B, -1).shape[1]
    w, mu, cv = _params(w, mu, cv, B, K, D, cov)
    nk = np.zeros((B, K))
    sx = np.zeros((B, K, D))
    sxx = np.zeros((B, cov_len(cov, D, K)))
    ll = np.zeros(B)
    flags = np.zeros((B, K), dtype=np.int32)
    rc = _load().oracle_estep(COV[cov], B, N, D, K, _ptr(Xa), xt, _ptr(w), _ptr(mu), _ptr(cv),
                              _ptr(nk), _ptr(sx), _ptr(sxx), _ptr(ll), _ptr(flags), int(nthreads))
    if rc:
        raise ValueError("oracle_estep rejected its arguments")
    return dict(nk=nk, sx=sx, sxx=sxx, ll=ll, flags=flags)


def mstep(cov, stats, n, w, mu, cv, eps=1e-6):
    """Parameters after the M-step.  Returns (w', mu', cv', flags)."""
    nk = np.ascontiguousarray(stats["nk"], dtype=np.float64)
    B, K = nk.shape
    D = stats["sx"].shape[2]
    w, mu, cv = _params(w, mu, cv, B, K, D, cov)
    sx = np.ascontiguousarray(stats["sx"], dtype=np.float64)
    sxx = np.ascontiguousarray(stats["sxx"], dtype=np.float64)
    wo, mo, co = np.zeros_like(w), np.zeros_like(mu), np.zeros_like(cv)
    flags = np.zeros((B, K), dtype=np.int32)
    rc = _load().oracle_mstep(COV[cov], B, int(n), D, K, _ptr(nk), _ptr(sx), _ptr(sxx),
                              _ptr(w), _ptr(mu), _ptr(cv), float(eps),
                              _ptr(wo), _ptr(mo), _ptr(co), _ptr(flags))
    if rc:
        raise ValueError("oracle_mstep rejected its arguments")
    return wo, mo, co, flags


def mstep_twopass(cov, X, w, mu, cv, eps=1e-6):
    """Literal two-pass M-step for one problem (cross-check of the identity)."""
    Xa, xt = _x_and_type(X)
    N, D = Xa.shape
    K = np.asarray(w).size
    w, mu, cv = (a[0] for a in _params(w, mu, cv, 1, K, D, cov))
    wo, mo, co = np.zeros_like(w), np.zeros_like(mu), np.zeros_like(cv)
    _load().oracle_mstep_twopass(COV[cov], N, D, K, _ptr(Xa), xt, _ptr(w), _ptr(mu), _ptr(cv),
                                 float(eps), _ptr(wo), _ptr(mo), _ptr(co))
    return wo, mo, co


def responsibilities(cov, X, w, mu, cv):
    """(logscore (N,K), r (N,K), lse (N)) for one problem (small N only)."""
    Xa, xt = _x_and_type(X)
    N, D = Xa.shape
    K = np.asarray(w).size
    w, mu, cv = (a[0] for a in _params(w, mu, cv, 1, K, D, cov))
    ls, r, lse = np.zeros((N, K)), np.zeros((N, K)), np.zeros(N)
    _load().oracle_responsibilities(COV[cov], N, D, K, _ptr(Xa), xt, _ptr(w), _ptr(mu), _ptr(cv),
                                    _ptr(ls), _ptr(r), _ptr(lse))
    return ls, r, lse


def topm(cov, X, w, mu, cv, m, thr, nthreads=0):
    """Soft multi-assignment for one problem: (idx, resp, count, logp, margin)."""
    Xa, xt = _x_and_type(X)
    N, D = Xa.shape
    K = np.asarray(w).size
    w, mu, cv = (a[0] for a in _params(w, mu, cv, 1, K, D, cov))
    idx = np.zeros((N, m), dtype=np.int32)
    resp = np.zeros((N, m))
    count = np.zeros(N, dtype=np.int32)
    logp = np.zeros(N)
    margin = np.zeros(N)
    rc = _load().oracle_topm(COV[cov], N, D, K, _ptr(Xa), xt, _ptr(w), _ptr(mu), _ptr(cv),
                             int(m), float(thr), _ptr(idx), _ptr(resp), _ptr(count), _ptr(logp),
                             _ptr(margin), int(nthreads))
    if rc:
        raise ValueError("oracle_topm rejected its arguments")
    return idx, resp, count, logp, margin


def fit_step(cov, X, w, mu, cv, eps=1e-6, nthreads=0):
    """One EM iteration theta_t -> theta_{t+1} (float64), with the mean LL of theta_t."""
    Xa, _ = _x_and_type(X)
    n = Xa.shape[-2]
    st = estep(cov, X, w, mu, cv, nthreads)
    B = st["nk"].shape[0]
    wo, mo, co, fl = mstep(cov, st, n, np.asarray(w).reshape(B, -1),
                           np.asarray(mu).reshape(st["sx"].shape), np.asarray(cv).reshape(st["sxx"].shape), eps)
    return dict(w=wo, mu=mo, cv=co, mean_ll=st["ll"] / n, stats=st, flags=fl)


def kmeans_step(X, C, nthreads=0):
    """One k-means (Lloyd) iteration for one problem from centroids C (K, D):
    (labels (N) int32, gap (N), new centroids (K, D), counts (K) int64,
    inertia).  gap = second smallest minus smallest squared distance of the
    row, the margin its label depends on."""
    Xa, xt = _x_and_type(X)
    N, D = Xa.shape
    C = np.ascontiguousarray(C, dtype=np.float64).reshape(-1, D)
    K = C.shape[0]
    labels = np.zeros(N, dtype=np.int32)
    gap = np.zeros(N)
    newC = np.zeros((K, D))
    counts = np.zeros(K, dtype=np.int64)
    inertia = np.zeros(1)
    rc = _load().oracle_kmeans_step(N, D, K, _ptr(Xa), xt, _ptr(C), _ptr(labels), _ptr(gap), _ptr(newC),
                                    _ptr(counts), _ptr(inertia), int(nthreads))
    if rc:
        raise ValueError("oracle_kmeans_step rejected its arguments")
    return labels, gap, newC, counts, float(inertia[0])


def ivf_lists(idx, resp, K):
    """Inverted lists (IVF posting lists) of a soft multi-assignment.

    "Flash-GMM: A Memory-Efficient Kernel for Scalable Soft Clustering",
    Section 4 (GMM as the IVF coarse quantizer, the multi-assignment scheme of
    Section 4.3) and Conclusion (boundary vectors are stored in several posting
    lists): row i of problem b goes into the list of every component that its
    multi-assignment kept.  idx (B,N,m) int32: a row's entries are its leading
    values in [0, K); the first value outside that range ends the row.  resp
    (B,N,m) float or None.  Lists hold rows in increasing row order (the pages
    fix no order; this is the plainest deterministic one).

    Returns offsets (B,K+1) int64 (list k of problem b is rows[b, offsets[b,k]
    : offsets[b,k+1]]), rows (B,N*m) int32 and list_resp (B,N*m) float32 (or
    None), both -1 / 0 past offsets[b,K].  Written as the definition, one row
    at a time: small inputs only.
    """
    idx = np.asarray(idx)
    B, N, m = idx.shape
    offsets = np.zeros((B, K + 1), np.int64)
    rows = np.full((B, N * m), -1, np.int32)
    lr = None if resp is None else np.zeros((B, N * m), np.float32)
    for b in range(B):
        lists = [[] for _ in range(K)]
        for i in range(N):
            for j in range(m):
                k = int(idx[b, i, j])
                if k < 0 or k >= K:
                    break
                lists[k].append((i, 0.0 if resp is None else float(resp[b, i, j])))
        pos = 0
        for k in range(K):
            offsets[b, k] = pos
            for i, r in lists[k]:
                rows[b, pos] = i
                if lr is not None:
                    lr[b, pos] = r
                pos += 1
        offsets[b, K] = pos
    return offsets, rows, lr


def fisher_vector(X, w, mu, var, power=True, l2=True):
    """Fisher vectors of B sets of rows under one diagonal GMM (w (K,), mu
    (K, D), var (K, D)): the application Flash-GMM's closing discussion names
    (Fisher Vector encoding, Perronnin et al. 2010), in its improved form.
    Per set of N rows, with r the responsibilities:
      G_mu[k, d]  = 1 / (N sqrt(w_k))   sum_i r_ik (x_id - mu_kd) / sigma_kd
      G_sig[k, d] = 1 / (N sqrt(2 w_k)) sum_i r_ik (((x_id - mu_kd) / sigma_kd)^2 - 1)
    (the gradients of the mean log-likelihood with respect to mu and sigma,
    scaled by the diagonal Fisher information), concatenated k-major as
    [G_mu, G_sig], then optionally a signed square root and L2 normalisation.
    Returns (B, 2 K D) float64."""
    X = np.asarray(X, dtype=np.float64)
    if X.ndim == 2:
        X = X[None]
    w = np.asarray(w, dtype=np.float64).reshape(-1)
    mu = np.asarray(mu, dtype=np.float64).reshape(w.size, -1)
    var = np.asarray(var, dtype=np.float64).reshape(mu.shape)
    sig = np.sqrt(var)
    out = []
    for Xb in X:
        N = Xb.shape[0]
        _, r, _ = responsibilities("diag", Xb, w, mu, var)
        z = (Xb[:, None, :] - mu[None]) / sig[None]  # (N, K, D)
        gmu = np.einsum("nk,nkd->kd", r, z) / (N * np.sqrt(w))[:, None]
        gsig = np.einsum("nk,nkd->kd", r, z * z - 1.0) / (N * np.sqrt(2.0 * w))[:, None]
        fv = np.concatenate([gmu.ravel(), gsig.ravel()])
        if power:
            fv = np.sign(fv) * np.sqrt(np.abs(fv))
        if l2:
            n = np.linalg.norm(fv)
            if n > 0:
                fv = fv / n
        out.append(fv)
    return np.stack(out)


def topk_fit_step(cov, X, w, mu, cv, topk, eps=1e-6):
    """One approximate top-k EM iteration for one problem (spherical or
    diagonal): the training mode the GMMXX README lists as approx_top_k
    ("Useful Options" and "CUDA backend (experimental)").  Each row keeps the
    topk components of largest log-score log pi_k N(x | theta_k) (ties to the
    lower index), normalises its responsibilities over that subset only, and
    only those enter the statistics; the M-step is the usual one.  With
    topk >= K every component is kept, which is the exact EM step.  Returns a
    dict like fit_step: w, mu, cv (each with a leading problem axis), mean_ll =
    the mean over rows of the log-sum-exp over each row's kept components, the
    statistics, and keep (N, topk) the kept components, best first, -1 past K."""
    Xa = decode_rows(X)
    N, D = Xa.shape
    ls, _, _ = responsibilities(cov, X, w, mu, cv)
    K = ls.shape[1]
    m = min(int(topk), K)
    order = np.argsort(-ls, axis=1, kind="stable")[:, :m]  # descending score, ties: lower index first
    sel = np.take_along_axis(ls, order, axis=1)
    mx = sel[:, :1]
    lse = (mx + np.log(np.exp(sel - mx).sum(axis=1, keepdims=True)))[:, 0]
    r = np.zeros((N, K))
    np.put_along_axis(r, order, np.exp(sel - lse[:, None]), axis=1)
    mu0 = np.asarray(mu, dtype=np.float64).reshape(K, D)
    nk = r.sum(axis=0)
    sx = r.T @ Xa
    diff2 = (Xa[:, None, :] - mu0[None]) ** 2  # (N, K, D)
    sxx = np.einsum("nk,nkd->kd", r, diff2)
    if cov == "spherical":
        sxx = sxx.sum(axis=1)
    st = dict(nk=nk[None], sx=sx[None], sxx=sxx[None], ll=np.array([lse.sum()]))
    wo, mo, co, fl = mstep(cov, st, N, np.asarray(w).reshape(1, K), mu0[None], np.asarray(cv).reshape(st["sxx"].shape), eps)
    keep = np.full((N, max(int(topk), 1)), -1, dtype=np.int64)
    keep[:, :m] = order
    return dict(w=wo, mu=mo, cv=co, mean_ll=np.array([lse.mean()]), stats=st, flags=fl, keep=keep)


def kde_score(Y, X, h):
    """Log of the Gaussian kernel density estimate at each query row: the
    other application Flash-GMM's closing discussion names beside Fisher
    vectors.  With M reference rows x_j and an isotropic bandwidth h, the
    estimate is a mixture of M equal-weight spherical Gaussians centred on the
    references with variance h^2:
      log p(y) = logsumexp_j(-|y - x_j|^2 / (2 h^2)) - log M - (D / 2) log(2 pi h^2).
    Squared distances by direct differences in float64.  Y: (N, D) or
    (B, N, D); X: (M, D).  Returns float64 of Y's leading shape."""
    from scipy.special import logsumexp
    Y = np.asarray(Y, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    lead = Y.shape[:-1]
    Y = Y.reshape(-1, Y.shape[-1])
    M, D = X.shape
    h = float(h)
    const = -np.log(M) - 0.5 * D * np.log(2.0 * np.pi * h * h)
    out = np.empty(Y.shape[0])
    step = max(1, int(2e7 // max(1, M * D)))
    for s in range(0, Y.shape[0], step):
        diff = Y[s:s + step, None, :] - X[None, :, :]
        d2 = np.einsum("nmd,nmd->nm", diff, diff)
        out[s:s + step] = logsumexp(-d2 / (2.0 * h * h), axis=1) + const
    return out.reshape(lead)
