"""Estimator-level calls over the C ABI: per-row log-likelihood, hard
assignment, mean log-likelihood, information criteria, and a fit loop with
restarts -- the estimator surface the GMMXX README lists under "Highlights"
(fit, predict, score, score_samples, aic, bic; restarts as in its estimator).

Every per-row and per-component number comes from the HIP library:
score_samples and predict from gmm_predict_proba_topm (m = 1: the best
component and log p(x_i)), score from gmm_estep_stats (sum_i log p(x_i)),
fit from gmm_fit_step (or gmm_topk_fit_step, the approximate top-k mode of
the GMMXX README), KernelDensity.score_samples from gmm_kde_score.  What runs
here is argument handling, the stopping rule and the AIC/BIC arithmetic on B
returned scalars.

  n_parameters(cov, K, D)                       -> int
  score_samples(X, w, mu, cv, cov)              -> (B, N) float32 log p(x_i)
  predict(X, w, mu, cv, cov)                    -> (B, N) int32 argmax_k r_ik
  score(X, w, mu, cv, cov)                      -> (B,) float64 mean log p(x_i)
  information_criteria(mean_ll, N, p)           -> (aic, bic), numpy
  aic(...), bic(...)                            -> (B,) float64
  fit(X, K, cov, ...)                           -> FitResult (the restart with the best mean LL)
  GaussianMixture(n_components, covariance_type, ...)  the same calls as a scikit-learn style class
  KMeans(n_clusters, ...)                       Lloyd iterations over gmm_kmeans_step (the hard limit)
  KernelDensity(bandwidth)                      Gaussian kernel density estimate over gmm_kde_score
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from . import (gmm_estep_stats, gmm_fit, gmm_fit_step, gmm_kde_score, gmm_kmeans_step, gmm_predict_proba_topm,
               gmm_topk_fit_step, gmm_topk_fit_workspace_bytes, new_stats)


def _torch():
    import torch
    return torch


def _batched(X):
    return X if X.dim() == 3 else X.unsqueeze(0)


def n_parameters(cov: str, K: int, D: int) -> int:
    """Free parameters of a K-component mixture in D dimensions: K - 1 weights,
    K D means, and the covariance parameters (spherical K, diag K D, tied
    D (D + 1) / 2, full K D (D + 1) / 2)."""
    covp = {"spherical": K, "diag": K * D, "tied": D * (D + 1) // 2, "full": K * D * (D + 1) // 2}[cov]
    return (K - 1) + K * D + covp


def information_criteria(mean_ll, N: int, p: int):
    """AIC = -2 N mean_ll + 2 p and BIC = -2 N mean_ll + p log N (Akaike;
    Schwarz), per problem."""
    total = -2.0 * np.asarray(mean_ll, dtype=np.float64) * N
    return total + 2.0 * p, total + p * math.log(N)


def _topm1(X, w, mu, cv, cov):
    torch = _torch()
    Xb = _batched(X)
    B, N = Xb.shape[0], Xb.shape[1]
    idx = torch.empty(B, N, 1, dtype=torch.int32, device=X.device)
    resp = torch.empty(B, N, 1, dtype=torch.float32, device=X.device)
    logp = torch.empty(B, N, dtype=torch.float32, device=X.device)
    gmm_predict_proba_topm(X, w, mu, cv, cov, 1, 0.0, idx, resp, logp=logp)
    return idx[..., 0], logp


def score_samples(X, w, mu, cv, cov):
    """log p(x_i) (natural log) of every row, (B, N) float32."""
    return _topm1(X, w, mu, cv, cov)[1]


def predict(X, w, mu, cv, cov):
    """The component of largest responsibility of every row (ties: lower
    index), (B, N) int32."""
    return _topm1(X, w, mu, cv, cov)[0]


def score(X, w, mu, cv, cov):
    """(1/N) sum_i log p(x_i) per problem, (B,) float64 on the host."""
    Xb = _batched(X)
    B, N, D = Xb.shape
    st = new_stats(B, w.shape[-1], D, cov, X.device)
    gmm_estep_stats(X, w, mu, cv, cov, st)
    return (st["loglik"] / N).cpu().numpy()


def aic(X, w, mu, cv, cov):
    Xb = _batched(X)
    return information_criteria(score(X, w, mu, cv, cov), Xb.shape[1], n_parameters(cov, w.shape[-1], Xb.shape[2]))[0]


def bic(X, w, mu, cv, cov):
    Xb = _batched(X)
    return information_criteria(score(X, w, mu, cv, cov), Xb.shape[1], n_parameters(cov, w.shape[-1], Xb.shape[2]))[1]


@dataclass
class FitResult:
    weights: object        # (B, K) float32, device
    means: object          # (B, K, D) float32, device
    covars: object         # covariance parameters, device
    mean_ll: np.ndarray    # (B,) mean log-likelihood of the returned parameters' last E-step
    n_iter: int
    converged: bool
    restart: int           # which restart was kept
    history: list          # per restart: list of per-iteration mean LL (problem-averaged)


def random_init(X, K, cov, generator):
    """K distinct rows of each problem as means, equal weights, and the
    problem's sample variance (spherical: its mean over dimensions; diag: per
    dimension; tied/full: the sample covariance) as every component's."""
    torch = _torch()
    Xb = _batched(X).float()
    B, N, D = Xb.shape
    if K > N:
        raise ValueError("K exceeds the number of rows")
    sel = torch.stack([torch.randperm(N, generator=generator, device="cpu")[:K] for _ in range(B)]).to(X.device)
    mu = torch.gather(Xb, 1, sel[..., None].expand(B, K, D)).contiguous()
    w = torch.full((B, K), 1.0 / K, dtype=torch.float32, device=X.device)
    xm = Xb.mean(dim=1, keepdim=True)
    var = ((Xb - xm) ** 2).mean(dim=1)  # (B, D)
    if cov == "spherical":
        cv = var.mean(dim=1, keepdim=True).expand(B, K).contiguous()
    elif cov == "diag":
        cv = var[:, None, :].expand(B, K, D).contiguous()
    else:
        Xc = (Xb - xm).contiguous()
        C = torch.bmm(Xc.transpose(1, 2).contiguous(), Xc) / N
        cv = C.contiguous() if cov == "tied" else C[:, None].expand(B, K, D, D).contiguous()
    if X.dim() == 2:
        w, mu, cv = w[0].contiguous(), mu[0].contiguous(), cv[0].contiguous()
    return w, mu, cv


def fit(X, K, cov, n_iter=100, tol=1e-3, n_init=1, reg_covar=1e-6, seed=0, init=None, topk=None, check_every=1):
    """EM from n_init starts (random_init with a seeded generator, or the
    given init = (w, mu, cv) for the first start); each runs until the change
    of the problem-averaged mean log-likelihood falls below tol or n_iter
    iterations.  Keeps the start whose last mean log-likelihood is highest.
    check_every: iterations per gmm_fit call between two reads of the
    log-likelihoods on the host (1: the test after every iteration, as above;
    c > 1: one synchronisation per c iterations, and up to c - 1 iterations
    past the one where the test first holds, which EM only improves; the
    history and n_iter still end at that iteration).
    topk: run approximate top-k EM steps instead (each row keeps its topk best
    components; spherical and diagonal covariance); the history then holds
    the top-k steps' log-likelihoods, the final score the full mixture's."""
    torch = _torch()
    tws = None
    if topk is not None:
        n = gmm_topk_fit_workspace_bytes(X, K, cov, int(topk))
        tws = torch.empty(max(n, 256), dtype=torch.uint8, device=X.device)
    gen = torch.Generator(device="cpu").manual_seed(seed)
    Xb = _batched(X)
    B = Xb.shape[0]
    best, history = None, []
    for r in range(n_init):
        if r == 0 and init is not None:
            w, mu, cv = (t.clone().contiguous() for t in init)
        else:
            w, mu, cv = random_init(X, K, cov, gen)
        hist, prev, converged, it = [], None, False, 0
        if topk is None and check_every > 1:
            # blocks of check_every iterations in one call each, their
            # log-likelihoods read once per block
            mlls = torch.zeros((int(check_every), B), dtype=torch.float64, device=X.device)
            done = 0
            while done < n_iter and not converged:
                c = min(int(check_every), n_iter - done)
                gmm_fit(X, w, mu, cv, cov, c, reg_covar=reg_covar, mean_loglik=mlls)
                for cur in mlls[:c].mean(dim=1).tolist():  # the LL entering each iteration
                    it += 1
                    hist.append(cur)
                    if prev is not None and abs(cur - prev) < tol:
                        converged = True
                        break
                    prev = cur
                done += c
        else:
            mll = torch.zeros(B, dtype=torch.float64, device=X.device)
            for it in range(1, n_iter + 1):
                if topk is None:
                    gmm_fit_step(X, w, mu, cv, cov, reg_covar=reg_covar, mean_loglik=mll)
                else:
                    gmm_topk_fit_step(X, w, mu, cv, cov, int(topk), reg_covar=reg_covar, mean_loglik=mll, ws=tws)
                cur = float(mll.mean().item())  # the LL of the parameters that entered this step
                hist.append(cur)
                if prev is not None and abs(cur - prev) < tol:
                    converged = True
                    break
                prev = cur
        history.append(hist)
        final = score(X, w, mu, cv, cov)
        if best is None or final.mean() > best.mean_ll.mean():
            best = FitResult(w, mu, cv, final, it, converged, r, history)
    best.history = history
    return best


class GaussianMixture:
    """The estimator in the scikit-learn style of the GMMXX README (its Python
    usage example): fit / predict / predict_proba_topm / score_samples /
    score / aic / bic, with the fitted state in means_, weights_,
    covariances_ (spherical (K,) variances, diag (K, D), tied (D, D), full
    (K, D, D)), lower_bound_ (the last E-step's mean log-likelihood),
    lower_bound_history_ (per iteration, kept restart), n_iter_ and
    converged_.  X is one problem, (N, D), on the GPU; the state stays on
    the GPU as float32 tensors.  Every computation runs in the HIP library."""

    def __init__(self, n_components, covariance_type="full", max_iter=100, tol=1e-3, reg_covar=1e-6, n_init=1,
                 random_state=0, weights_init=None, means_init=None, covariances_init=None, init_params="random",
                 topk=None, check_every=1):
        if covariance_type not in ("spherical", "diag", "tied", "full"):
            raise ValueError(f"unknown covariance_type {covariance_type!r}")
        if init_params not in ("random", "kmeans"):
            raise ValueError(f"unknown init_params {init_params!r}")
        self.init_params = init_params
        self.topk = None if topk is None else int(topk)
        self.check_every = max(1, int(check_every))  # iterations per host read of the log-likelihood
        self.n_components = int(n_components)
        self.covariance_type = covariance_type
        self.max_iter = int(max_iter)
        self.tol = float(tol)
        self.reg_covar = float(reg_covar)
        self.n_init = int(n_init)
        self.random_state = random_state
        self.weights_init, self.means_init, self.covariances_init = weights_init, means_init, covariances_init

    def _init(self, X):
        given = (self.weights_init, self.means_init, self.covariances_init)
        if all(t is None for t in given):
            return self._kmeans_init(X) if self.init_params == "kmeans" else None
        if any(t is None for t in given):
            raise ValueError("weights_init, means_init and covariances_init are given together")
        torch = _torch()
        return tuple(torch.as_tensor(t, dtype=torch.float32, device=X.device).contiguous() for t in given)

    def _kmeans_init(self, X):
        """Means from Lloyd iterations (KMeans with this seed), weights from the
        cluster sizes (at least one row each), and the covariance of
        random_init (the data's variance) for every component."""
        torch = _torch()
        km = KMeans(self.n_components, max_iter=20, random_state=self.random_state).fit(X)
        gen = torch.Generator(device="cpu").manual_seed(int(self.random_state or 0))
        _, _, cv = random_init(X, self.n_components, self.covariance_type, gen)
        cnt = km.counts_.to(torch.float64).clamp_min(1.0)
        w = (cnt / cnt.sum()).to(torch.float32).contiguous()
        return w, km.cluster_centers_.clone().contiguous(), cv

    def fit(self, X):
        if X.dim() != 2:
            raise ValueError("X is (N, D)")
        res = fit(X, self.n_components, self.covariance_type, n_iter=self.max_iter, tol=self.tol,
                  n_init=self.n_init, reg_covar=self.reg_covar, seed=self.random_state or 0, init=self._init(X),
                  topk=self.topk, check_every=self.check_every)
        self.weights_, self.means_, self.covariances_ = res.weights, res.means, res.covars
        self.lower_bound_ = float(res.mean_ll[0])
        self.lower_bound_history_ = list(res.history[res.restart])
        self.n_iter_, self.converged_ = res.n_iter, res.converged
        self.n_features_in_ = int(X.shape[1])
        return self

    def _theta(self):
        if not hasattr(self, "means_"):
            raise RuntimeError("call fit first")
        return self.weights_, self.means_, self.covariances_, self.covariance_type

    def fit_predict(self, X):
        return self.fit(X).predict(X)

    def predict(self, X):
        return predict(X, *self._theta())[0]

    def score_samples(self, X):
        return score_samples(X, *self._theta())[0]

    def score(self, X):
        return float(score(X, *self._theta())[0])

    def aic(self, X):
        return float(aic(X, *self._theta())[0])

    def bic(self, X):
        return float(bic(X, *self._theta())[0])

    def predict_proba_topm(self, X, m=4, threshold=0.1):
        """Soft multi-assignment: per row the components of the m largest
        responsibilities that reach threshold (the largest always kept),
        in descending order with ties to the lower index.  Returns idx (N, m)
        int32 (-1 past count), resp (N, m) float32, count (N,) int32."""
        torch = _torch()
        N = X.shape[0]
        idx = torch.empty(N, m, dtype=torch.int32, device=X.device)
        resp = torch.empty(N, m, dtype=torch.float32, device=X.device)
        count = torch.empty(N, dtype=torch.int32, device=X.device)
        gmm_predict_proba_topm(X, *self._theta(), m, threshold, idx, resp, count=count)
        return idx, resp, count


class KMeans:
    """k-means by Lloyd iterations, each one gmm_kmeans_step (nearest
    centroid on float64 distances, cluster means summed in float64): the
    hard-assignment, shared-variance-to-zero limit of the GMM, and the usual
    IVF coarse quantizer the GMM replaces.  X is one problem, (N, D) float32
    or bfloat16, on the GPU.  Starts from K distinct rows drawn with the seed
    (or init, (K, D)); stops when the inertia falls by less than tol of
    itself, or after max_iter steps.  Fitted state (scikit-learn names):
    cluster_centers_ (K, D) float32, labels_ (N,) int32 and inertia_ under
    the final centres, counts_ (K,) int64, n_iter_, inertia_history_ (the
    inertia under the centres entering each step)."""

    def __init__(self, n_clusters, max_iter=100, tol=1e-4, random_state=0, init=None):
        self.n_clusters = int(n_clusters)
        self.max_iter = int(max_iter)
        self.tol = float(tol)
        self.random_state = random_state
        self.init = init

    def _start(self, X):
        torch = _torch()
        N, K = X.shape[0], self.n_clusters
        if self.init is not None:
            return torch.as_tensor(self.init, dtype=torch.float32, device=X.device).clone().contiguous()
        if K > N:
            raise ValueError("n_clusters exceeds the number of rows")
        gen = torch.Generator(device="cpu").manual_seed(int(self.random_state or 0))
        sel = torch.randperm(N, generator=gen)[:K].to(X.device)
        return X.index_select(0, sel).float().contiguous()

    def fit(self, X):
        if X.dim() != 2:
            raise ValueError("X is (N, D)")
        C = self._start(X)
        hist, it = [], 0
        for it in range(1, self.max_iter + 1):
            _, counts, inertia = gmm_kmeans_step(X, C)
            cur = float(inertia[0].item())
            hist.append(cur)
            if len(hist) > 1 and hist[-2] - cur <= self.tol * hist[-2]:
                break
        self.cluster_centers_ = C
        self.n_iter_ = it
        self.inertia_history_ = hist
        self.labels_, self.counts_, self.inertia_ = self._assign(X)
        return self

    def _assign(self, X):
        if not hasattr(self, "cluster_centers_"):
            raise RuntimeError("call fit first")
        labels, counts, inertia = gmm_kmeans_step(X, self.cluster_centers_.clone())
        return labels[0], counts[0], float(inertia[0].item())

    def predict(self, X):
        """The nearest centre of every row (ties: lower index), (N,) int32."""
        return self._assign(X)[0]

    def fit_predict(self, X):
        return self.fit(X).labels_


class KernelDensity:
    """Gaussian kernel density estimate in the scikit-learn style
    (KernelDensity(kernel="gaussian")): fit(X) keeps the reference rows (M, D)
    float32 on the GPU; score_samples(Y) is log p(y) per query row from
    gmm_kde_score; score(Y) their sum."""

    def __init__(self, bandwidth=1.0):
        if not (float(bandwidth) > 0.0):
            raise ValueError("bandwidth must be > 0")
        self.bandwidth = float(bandwidth)

    def fit(self, X):
        torch = _torch()
        if X.dim() != 2:
            raise ValueError("X is (M, D)")
        self.reference_ = X.to(torch.float32).contiguous()
        self.n_features_in_ = int(X.shape[1])
        return self

    def score_samples(self, Y):
        if not hasattr(self, "reference_"):
            raise RuntimeError("call fit first")
        return gmm_kde_score(Y.contiguous(), self.reference_, self.bandwidth)

    def score(self, Y):
        return float(self.score_samples(Y).double().sum().item())

