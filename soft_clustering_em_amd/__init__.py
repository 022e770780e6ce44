"""MI355X-native fused EM for Gaussian mixture models.

Python names mirror the C ABI of include/gmm.h.  They take torch tensors that
live on the GPU, fill the descriptor structs and call libgmm.so on the current
torch stream; every step of the computation runs in the HIP kernels.

  gmm_workspace_bytes(X, K, cov, op)          -> int
  gmm_estep_stats(X, w, mu, cv, stats, accumulate=False, ws=None)
  gmm_mstep(stats, n_total, w, mu, cv, reg_covar=1e-6, comp_status=None)
  gmm_fit_step(X, w, mu, cv, reg_covar=1e-6, mean_loglik=None, comp_status=None, ws=None)
  gmm_fit(X, w, mu, cv, cov, n_iter, reg_covar=1e-6, mean_loglik=None, comp_status=None, ws=None)
  gmm_fit_step_noalloc(X, w, mu, cv, cov, reg_covar=1e-6, mean_loglik=None, comp_status=None)
  gmm_fit_step_streamed(X_host, w, mu, cv, cov, chunk_rows, reg_covar=1e-6, mean_loglik=None,
                        comp_status=None, ws=None, copy_stream=None)   (rows stay in host memory)
  gmm_predict_proba_topm(X, w, mu, cv, m, threshold, idx, resp, count=None, logp=None, ws=None)
  gmm_ivf_lists(idx, K, resp=None, offsets=None, rows=None, list_resp=None, ws=None)
  gmm_kmeans_workspace_bytes(X, K)            -> int
  gmm_kmeans_step(X, centroids, labels=None, counts=None, inertia=None, ws=None)
  gmm_fisher_vector(X, w, mu, var, power=True, l2=True, fv=None, ws=None)
  gmm_topk_fit_step(X, w, mu, cv, cov, topk, reg_covar=1e-6, mean_loglik=None, comp_status=None, ws=None)
  gmm_check_components(comp_status)          -> (status, first index or -1); synchronises

The estimator calls (score_samples, predict, score, aic, bic, fit with
restarts) are in soft_clustering_em_amd.estimator.

X is (N, D) or (B, N, D) with unit stride along D; w (B,K), mu (B,K,D) and the
covariance parameters are float32 and are updated in place by the M-step.
"""
from __future__ import annotations

import ctypes

from . import _abi
from ._abi import (COV_CODES, GmmError, GmmData, GmmOptions, GmmParams, GmmStats, OP_ESTEP, OP_FIT,
                   OP_TOPM)

__all__ = ["gmm_workspace_bytes", "gmm_estep_stats", "gmm_mstep", "gmm_fit_step",
           "gmm_predict_proba_topm", "gmm_ivf_workspace_bytes", "gmm_ivf_lists", "gmm_kmeans_workspace_bytes",
           "gmm_kmeans_step", "gmm_fisher_vector_workspace_bytes", "gmm_fisher_vector",
           "gmm_topk_fit_workspace_bytes", "gmm_topk_fit_step", "new_stats", "GmmError",
           "cov_shape"]


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    return {torch.float32: _abi.DT_F32, torch.bfloat16: _abi.DT_BF16, torch.float16: _abi.DT_F16}[t.dtype]


def _data(X) -> GmmData:
    if X.dim() == 2:
        B, (N, D) = 1, X.shape
        ld, sb = X.stride(0), N * X.stride(0)
    elif X.dim() == 3:
        B, N, D = X.shape
        ld, sb = X.stride(1), X.stride(0)
    else:
        raise ValueError("X must be (N, D) or (B, N, D)")
    if D > 0 and N > 0 and X.stride(-1) != 1:
        raise ValueError("X needs unit stride along D")
    return GmmData(ctypes.c_void_p(X.data_ptr()), _dtype_code(X), B, N, D, ld, sb)


def _cov_code(cov):
    return COV_CODES[cov] if isinstance(cov, str) else int(cov)


def cov_shape(cov, B, K, D):
    return {"spherical": (B, K), "diag": (B, K, D), "tied": (B, D, D), "full": (B, K, D, D)}[cov]


def _params(w, mu, cv, cov) -> GmmParams:
    for t in (w, mu, cv):
        if not t.is_contiguous():
            raise ValueError("parameter tensors must be contiguous")
    K = w.shape[-1]
    return GmmParams(K, _cov_code(cov), ctypes.c_void_p(w.data_ptr()), ctypes.c_void_p(mu.data_ptr()),
                     ctypes.c_void_p(cv.data_ptr()))


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def gmm_workspace_bytes(X, K, cov, op=OP_FIT, m=0) -> int:
    d = _data(X)
    return int(_abi.lib().gmm_workspace_bytes(ctypes.byref(d), int(K), _cov_code(cov), int(op), int(m)))


def _workspace(X, K, cov, op, m, ws):
    if ws is not None:
        return ws
    torch = _torch()
    n = gmm_workspace_bytes(X, K, cov, op, m)
    if n == 0:
        # let the compute call report the precise reason
        return torch.empty(256, dtype=torch.uint8, device=X.device)
    return torch.empty(n, dtype=torch.uint8, device=X.device)


def new_stats(B, K, D, cov, device):
    """Zeroed float64 statistics buffers (nk, sx, sxx, loglik) for gmm_estep_stats."""
    torch = _torch()
    return dict(nk=torch.zeros(B, K, dtype=torch.float64, device=device),
                sx=torch.zeros(B, K, D, dtype=torch.float64, device=device),
                sxx=torch.zeros(cov_shape(cov, B, K, D), dtype=torch.float64, device=device),
                loglik=torch.zeros(B, dtype=torch.float64, device=device))


def gmm_estep_stats(X, w, mu, cv, cov, stats, accumulate=False, ws=None, stream=None):
    d = _data(X)
    p = _params(w, mu, cv, cov)
    st = GmmStats(_ptr(stats["nk"]), _ptr(stats["sx"]), _ptr(stats["sxx"]), _ptr(stats["loglik"]))
    ws = _workspace(X, p.K, cov, OP_ESTEP, 0, ws)
    _abi.check(_abi.lib().gmm_estep_stats(ctypes.byref(d), ctypes.byref(p), ctypes.byref(st),
                                          int(bool(accumulate)), _ptr(ws), ws.numel(), _stream(stream)))
    return stats


def gmm_mstep(stats, n_total, w, mu, cv, cov, reg_covar=1e-6, comp_status=None, stream=None):
    B, K, D = stats["sx"].shape
    p = _params(w, mu, cv, cov)
    st = GmmStats(_ptr(stats["nk"]), _ptr(stats["sx"]), _ptr(stats["sxx"]), _ptr(stats["loglik"]))
    o = GmmOptions(float(reg_covar), 0, None, None)
    _abi.check(_abi.lib().gmm_mstep(B, D, ctypes.byref(st), int(n_total), ctypes.byref(p), ctypes.byref(o),
                                    _ptr(comp_status), _stream(stream)))


def gmm_fit_step(X, w, mu, cv, cov, reg_covar=1e-6, mean_loglik=None, comp_status=None, ws=None,
                 stream=None, events=None):
    """One EM iteration in place.  events: optional (begin, end) torch.cuda.Event
    pair recorded around the fused E-step kernel."""
    d = _data(X)
    p = _params(w, mu, cv, cov)
    eb = ee = None
    if events is not None:
        eb, ee = (ctypes.c_void_p(e.cuda_event) for e in events)
    o = GmmOptions(float(reg_covar), 0, eb, ee)
    ws = _workspace(X, p.K, cov, OP_FIT, 0, ws)
    _abi.check(_abi.lib().gmm_fit_step(ctypes.byref(d), ctypes.byref(p), ctypes.byref(o), _ptr(mean_loglik),
                                       _ptr(comp_status), _ptr(ws), ws.numel(), _stream(stream)))


def gmm_fit(X, w, mu, cv, cov, n_iter, reg_covar=1e-6, mean_loglik=None, comp_status=None, ws=None, stream=None,
            events=None):
    """n_iter EM iterations in place, the results of n_iter gmm_fit_step calls.
    mean_loglik: optional (n_iter, B) float64 device tensor, row t the mean
    log-likelihood entering iteration t.  events: optional (begin, end) pair
    recorded around the last iteration's E-step."""
    d = _data(X)
    p = _params(w, mu, cv, cov)
    if mean_loglik is not None:
        import torch
        if (mean_loglik.dtype != torch.float64 or not mean_loglik.is_cuda or not mean_loglik.is_contiguous()
                or mean_loglik.numel() < int(n_iter) * int(d.B)):
            raise ValueError("mean_loglik must be a contiguous float64 device tensor of n_iter * B elements")
    eb = ee = None
    if events is not None:
        eb, ee = (ctypes.c_void_p(e.cuda_event) for e in events)
    o = GmmOptions(float(reg_covar), 0, eb, ee)
    ws = _workspace(X, p.K, cov, OP_FIT, 0, ws)
    _abi.check(_abi.lib().gmm_fit(ctypes.byref(d), ctypes.byref(p), ctypes.byref(o), int(n_iter),
                                  _ptr(mean_loglik), _ptr(comp_status), _ptr(ws), ws.numel(), _stream(stream)))


def gmm_fit_step_noalloc(X, w, mu, cv, cov, reg_covar=1e-6, mean_loglik=None, comp_status=None, stream=None):
    """One EM iteration in place, with the library's static scratch array
    instead of a workspace (nothing is allocated on the device)."""
    d = _data(X)
    p = _params(w, mu, cv, cov)
    o = GmmOptions(float(reg_covar), 0, None, None)
    _abi.check(_abi.lib().gmm_fit_step_noalloc(ctypes.byref(d), ctypes.byref(p), ctypes.byref(o),
                                               _ptr(mean_loglik), _ptr(comp_status), _stream(stream)))


def gmm_fit_step_streamed_workspace_bytes(X_host, K, cov, chunk_rows) -> int:
    d = _data(X_host)
    return int(_abi.lib().gmm_fit_step_streamed_workspace_bytes(ctypes.byref(d), int(K), _cov_code(cov),
                                                                int(chunk_rows)))


def gmm_fit_step_streamed(X_host, w, mu, cv, cov, chunk_rows, reg_covar=1e-6, mean_loglik=None, comp_status=None,
                          ws=None, stream=None, copy_stream=None):
    """One EM iteration in place over rows in host memory (X_host: a CPU
    tensor, pinned for overlapped copies), streamed through two device chunk
    buffers of chunk_rows rows; copy_stream: a torch.cuda.Stream for the
    copies (None: the compute stream)."""
    torch = _torch()
    if X_host.is_cuda:
        raise ValueError("gmm_fit_step_streamed takes rows in host memory")
    d = _data(X_host)
    p = _params(w, mu, cv, cov)
    o = GmmOptions(float(reg_covar), 0, None, None)
    if ws is None:
        n = gmm_fit_step_streamed_workspace_bytes(X_host, p.K, cov, chunk_rows)
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device=w.device)
    cs = None if copy_stream is None else ctypes.c_void_p(copy_stream.cuda_stream)
    _abi.check(_abi.lib().gmm_fit_step_streamed(ctypes.byref(d), ctypes.byref(p), ctypes.byref(o), int(chunk_rows),
                                                _ptr(mean_loglik), _ptr(comp_status), _ptr(ws), ws.numel(),
                                                _stream(stream), cs))


def gmm_predict_proba_topm(X, w, mu, cv, cov, m, threshold, idx, resp, count=None, logp=None, ws=None,
                           stream=None):
    d = _data(X)
    p = _params(w, mu, cv, cov)
    ws = _workspace(X, p.K, cov, OP_TOPM, m, ws)
    _abi.check(_abi.lib().gmm_predict_proba_topm(ctypes.byref(d), ctypes.byref(p), int(m), float(threshold),
                                                 _ptr(idx), _ptr(resp), _ptr(count), _ptr(logp), _ptr(ws),
                                                 ws.numel(), _stream(stream)))


def gmm_ivf_workspace_bytes(B, N, m, K) -> int:
    return int(_abi.lib().gmm_ivf_workspace_bytes(int(B), int(N), int(m), int(K)))


def gmm_ivf_lists(idx, K, resp=None, offsets=None, rows=None, list_resp=None, ws=None, stream=None):
    """Posting lists of a multi-assignment idx ((N, m) or (B, N, m) int32 on the GPU).

    Returns (offsets (B, K+1) int64, rows (B, N*m) int32, list_resp (B, N*m) float32 or None);
    outputs not given are allocated here (rows and list_resp past offsets[b, K] are left as
    allocated)."""
    torch = _torch()
    if idx.dim() == 2:
        idx = idx.unsqueeze(0)
        resp = resp.unsqueeze(0) if resp is not None else None
    if not idx.is_contiguous() or idx.dtype != torch.int32:
        raise ValueError("idx must be a contiguous int32 tensor")
    if resp is not None and (not resp.is_contiguous() or resp.dtype != torch.float32 or resp.shape != idx.shape):
        raise ValueError("resp must be a contiguous float32 tensor shaped like idx")
    B, N, m = idx.shape
    dev = idx.device
    if offsets is None:
        offsets = torch.empty(B, K + 1, dtype=torch.int64, device=dev)
    if rows is None:
        rows = torch.empty(B, N * m, dtype=torch.int32, device=dev)
    if list_resp is None and resp is not None:
        list_resp = torch.empty(B, N * m, dtype=torch.float32, device=dev)
    if ws is None:
        n = gmm_ivf_workspace_bytes(B, N, m, K)
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
    _abi.check(_abi.lib().gmm_ivf_lists(int(B), int(N), int(m), int(K), _ptr(idx), _ptr(resp), _ptr(offsets),
                                        _ptr(rows), _ptr(list_resp), _ptr(ws), ws.numel(), _stream(stream)))
    return offsets, rows, list_resp


def gmm_kmeans_workspace_bytes(X, K) -> int:
    d = _data(X)
    return int(_abi.lib().gmm_kmeans_workspace_bytes(ctypes.byref(d), int(K)))


def gmm_kmeans_step(X, centroids, labels=None, counts=None, inertia=None, ws=None, stream=None):
    """One k-means (Lloyd) iteration; centroids ((K, D) or (B, K, D) float32)
    are replaced by the cluster means.  Returns (labels (B, N) int32 under the
    entering centroids, counts (B, K) int64, inertia (B,) float64); outputs
    not given are allocated here."""
    torch = _torch()
    d = _data(X)
    B, N = int(d.B), int(d.N)
    K = centroids.shape[-2]
    if centroids.dtype != torch.float32 or not centroids.is_contiguous() or centroids.numel() != B * K * d.D:
        raise ValueError("centroids must be a contiguous float32 tensor of B*K*D elements")
    dev = centroids.device
    if labels is None:
        labels = torch.empty(B, N, dtype=torch.int32, device=dev)
    if counts is None:
        counts = torch.empty(B, K, dtype=torch.int64, device=dev)
    if inertia is None:
        inertia = torch.empty(B, dtype=torch.float64, device=dev)
    if ws is None:
        n = gmm_kmeans_workspace_bytes(X, K)
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
    _abi.check(_abi.lib().gmm_kmeans_step(ctypes.byref(d), int(K), _ptr(centroids), _ptr(labels), _ptr(counts),
                                          _ptr(inertia), _ptr(ws), ws.numel(), _stream(stream)))
    return labels, counts, inertia


def gmm_fisher_vector_workspace_bytes(X, K) -> int:
    d = _data(X)
    return int(_abi.lib().gmm_fisher_vector_workspace_bytes(ctypes.byref(d), int(K)))


def gmm_fisher_vector(X, w, mu, var, power=True, l2=True, fv=None, ws=None, stream=None):
    """Fisher vectors of the sets X ((N, D) or (B, N, D) float32) under one
    diagonal model (w (K,), mu (K, D), var (K, D) float32): (B, 2 K D)
    float32, [G_mu, G_sigma] per set, optionally with the signed square root
    (power) and L2 normalisation."""
    torch = _torch()
    d = _data(X)
    B, K, D = int(d.B), int(w.shape[-1]), int(d.D)
    if mu.numel() != K * D or var.numel() != K * D:
        raise ValueError("the model is one diagonal GMM: w (K,), mu and var (K, D)")
    p = GmmParams(K, COV_CODES["diag"], ctypes.c_void_p(w.data_ptr()), ctypes.c_void_p(mu.data_ptr()),
                  ctypes.c_void_p(var.data_ptr()))
    if fv is None:
        fv = torch.empty(B, 2 * K * D, dtype=torch.float32, device=w.device)
    if ws is None:
        n = gmm_fisher_vector_workspace_bytes(X, K)
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device=w.device)
    flags = (1 if power else 0) | (2 if l2 else 0)
    _abi.check(_abi.lib().gmm_fisher_vector(ctypes.byref(d), ctypes.byref(p), flags, _ptr(fv), _ptr(ws), ws.numel(),
                                            _stream(stream)))
    return fv


def gmm_topk_fit_workspace_bytes(X, K, cov, topk) -> int:
    d = _data(X)
    return int(_abi.lib().gmm_topk_fit_workspace_bytes(ctypes.byref(d), int(K), _cov_code(cov), int(topk)))


def gmm_kde_workspace_bytes(Y, M) -> int:
    d = _data(Y)
    return int(_abi.lib().gmm_kde_workspace_bytes(ctypes.byref(d), int(M)))


def gmm_kde_score(Y, ref, bandwidth, out=None, ws=None, stream=None):
    """Log of the Gaussian kernel density estimate with bandwidth h over the
    reference rows ref ((M, D) float32) at the query rows Y ((N, D) or
    (B, N, D) float32): float32 of Y's leading shape."""
    torch = _torch()
    d = _data(Y)
    if ref.dim() != 2 or ref.shape[1] != d.D or ref.dtype != torch.float32:
        raise ValueError("ref must be (M, D) float32 with the queries' D")
    if ref.shape[0] > 0 and ref.stride(1) != 1:
        raise ValueError("ref needs unit stride along D")
    M = int(ref.shape[0])
    if out is None:
        out = torch.empty(Y.shape[:-1], dtype=torch.float32, device=Y.device)
    if ws is None:
        n = gmm_kde_workspace_bytes(Y, M)
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device=Y.device)
    _abi.check(_abi.lib().gmm_kde_score(ctypes.byref(d), _ptr(ref), M, int(ref.stride(0)), float(bandwidth), _ptr(out),
                                        _ptr(ws), ws.numel(), _stream(stream)))
    return out


def gmm_topk_fit_step(X, w, mu, cv, cov, topk, reg_covar=1e-6, mean_loglik=None, comp_status=None, ws=None,
                      stream=None):
    """One approximate top-k EM iteration in place (each row keeps its topk
    best components and normalises over them)."""
    torch = _torch()
    d = _data(X)
    p = _params(w, mu, cv, cov)
    o = GmmOptions(float(reg_covar), 0, None, None)
    if ws is None:
        n = gmm_topk_fit_workspace_bytes(X, p.K, cov, topk)
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device=X.device)
    _abi.check(_abi.lib().gmm_topk_fit_step(ctypes.byref(d), ctypes.byref(p), int(topk), ctypes.byref(o),
                                            _ptr(mean_loglik), _ptr(comp_status), _ptr(ws), ws.numel(),
                                            _stream(stream)))


def gmm_check_components(comp_status):
    """Copy comp_status (B, K) to the host (a synchronisation) and summarise it
    with the library's gmm_check_components: (GMM_ERR_NOT_PD, index of the
    first component whose input or updated covariance was not positive
    definite) or (GMM_OK, -1)."""
    import numpy as np
    host = np.ascontiguousarray(comp_status.detach().to("cpu").numpy(), dtype=np.int32).reshape(-1)
    first = ctypes.c_int64(-1)
    st = _abi.lib().gmm_check_components(host.ctypes.data, host.size, ctypes.byref(first))
    if st not in (_abi.GMM_OK, _abi.GMM_ERR_NOT_PD):
        _abi.check(st)
    return st, first.value
