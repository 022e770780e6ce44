"""GPU parity of the estimator calls (soft_clustering_em_amd.estimator)
against the oracle: per-row log p(x_i), the argmax component, the mean
log-likelihood, AIC/BIC, and the restart loop of fit()."""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import soft_clustering_em_amd._abi as abi
    abi.lib()
    return torch


def _theta(rng, cov, N, D, K):
    X = (rng.normal(size=(N, D)) + 4.0 * rng.integers(0, K, size=(N, 1)) * rng.normal(size=(1, D))).astype(np.float32)
    w = rng.dirichlet(np.full(K, 3.0)).astype(np.float32)
    mu = X[rng.choice(N, K, replace=False)].copy()
    if cov == "spherical":
        cv = rng.uniform(0.5, 2.0, size=K).astype(np.float32)
    elif cov == "diag":
        cv = rng.uniform(0.5, 2.0, size=(K, D)).astype(np.float32)
    elif cov == "tied":
        A = rng.normal(size=(D, D))
        cv = (A @ A.T / D + np.eye(D)).astype(np.float32)
    else:
        A = rng.normal(size=(K, D, D))
        cv = (A @ A.transpose(0, 2, 1) / D + np.eye(D)).astype(np.float32)
    return X, w, mu, cv


@pytest.mark.parametrize("cov,N,D,K", [("spherical", 5000, 8, 16), ("diag", 3001, 24, 40),
                                       ("tied", 2000, 6, 9), ("full", 2048, 16, 32),
                                       ("diag", 4000, 20, 600),        # E-step in blocks, exact top-m
                                       ("spherical", 3000, 128, 300)])
def test_score_samples_predict_score(torch_cuda, cov, N, D, K):
    from soft_clustering_em_amd import estimator as est
    torch = torch_cuda
    rng = np.random.default_rng(N + D + K)
    X, w, mu, cv = _theta(rng, cov, N, D, K)
    tX, tw, tmu, tcv = (torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (X, w, mu, cv))
    logp = est.score_samples(tX, tw, tmu, tcv, cov).cpu().numpy()[0]
    lab = est.predict(tX, tw, tmu, tcv, cov).cpu().numpy()[0]
    s = est.score(tX, tw, tmu, tcv, cov)[0]
    a, b = est.aic(tX, tw, tmu, tcv, cov)[0], est.bic(tX, tw, tmu, tcv, cov)[0]
    _, r, lse = oracle.responsibilities(cov, X, w, mu, cv)
    idx, _, _, _, margin = oracle.topm(cov, X, w, mu, cv, 1, 0.0)
    e_lp = float(np.max(np.abs(logp - lse) / np.maximum(1.0, np.abs(lse))))
    ok = margin > 1e-6
    print(f"{cov}: logp err {e_lp:.2e}, argmax rows checked {ok.sum()}/{N}", flush=True)
    assert e_lp <= 1e-5
    assert np.array_equal(lab[ok], idx[ok, 0])
    ll = lse.mean()
    assert abs(s - ll) <= 1e-6 * abs(ll)
    a_ref, b_ref = est.information_criteria(ll, N, est.n_parameters(cov, K, D))
    assert abs(a - a_ref) <= 1e-6 * abs(a_ref) and abs(b - b_ref) <= 1e-6 * abs(b_ref)


def test_fit_keeps_the_best_restart_and_ascends(torch_cuda):
    """Three restarts on the small spherical workload: each restart's mean
    log-likelihood never falls by more than float32 parameter rounding, and
    the kept restart has the highest final score of the three."""
    from soft_clustering_em_amd import estimator as est
    from soft_clustering_em_amd import synth
    torch = torch_cuda
    wl = synth.spherical_small()
    X = torch.from_numpy(wl.X[0]).cuda()
    res = est.fit(X, wl.K, "spherical", n_iter=15, tol=0.0, n_init=3, seed=1)
    finals = []
    for h in res.history:
        h = np.asarray(h)
        assert (np.diff(h) >= -1e-6 * np.abs(h[1:])).all(), h
        finals.append(h[-1])
    print("restart finals", finals, "kept", res.restart, flush=True)
    # the kept one scores at least as well as every restart's last recorded LL
    assert res.mean_ll.mean() >= max(finals) - 1e-6 * abs(max(finals))
    assert len(res.history) == 3 and res.n_iter == 15


def test_fit_in_blocks_matches_fit_per_iteration(torch_cuda):
    """check_every = 4 (gmm_fit blocks, one host read per block) gives the
    same history up to the converged iteration, and parameters that are the
    per-iteration fit's after the block's extra iterations (checked against
    gmm_fit_step from the same init, bit for bit)."""
    import soft_clustering_em_amd as g
    from soft_clustering_em_amd import estimator as est
    from soft_clustering_em_amd import synth
    torch = torch_cuda
    wl = synth.spherical_small()
    X = torch.from_numpy(wl.X[0]).cuda()
    init = tuple(torch.from_numpy(np.ascontiguousarray(a[0])).cuda() for a in (wl.w0, wl.mu0, wl.cv0))
    one = est.fit(X, wl.K, "spherical", n_iter=30, tol=1e-4, n_init=1, init=init)
    blk = est.fit(X, wl.K, "spherical", n_iter=30, tol=1e-4, n_init=1, init=init, check_every=4)
    assert blk.history[0] == one.history[0] and blk.n_iter == one.n_iter and blk.converged == one.converged
    ran = min(-(-blk.n_iter // 4) * 4, 30) if blk.converged else 30  # iterations the blocks ran
    w, mu, cv = (t.clone() for t in init)
    for _ in range(ran):
        g.gmm_fit_step(X, w, mu, cv, "spherical", reg_covar=1e-6)
    torch.cuda.synchronize()
    assert torch.equal(w, blk.weights) and torch.equal(mu, blk.means) and torch.equal(cv, blk.covars)


def test_fit_from_given_init_follows_the_oracle(torch_cuda):
    """fit() from an explicit init runs the same steps as the oracle from
    that init (first three iterations, one-step parity at 1e-4)."""
    from soft_clustering_em_amd import estimator as est
    from soft_clustering_em_amd import synth
    torch = torch_cuda
    wl = synth.spherical_small()
    X = torch.from_numpy(wl.X[0]).cuda()
    init = tuple(torch.from_numpy(np.ascontiguousarray(a[0])).cuda() for a in (wl.w0, wl.mu0, wl.cv0))
    res = est.fit(X, wl.K, "spherical", n_iter=3, tol=0.0, n_init=1, init=init)
    w, mu, cv = wl.w0[0].astype(np.float64), wl.mu0[0].astype(np.float64), wl.cv0[0].astype(np.float64)
    for _ in range(3):
        out = oracle.fit_step("spherical", wl.X[0], w, mu, cv)
        w, mu, cv = (out[k][0].astype(np.float32).astype(np.float64) for k in ("w", "mu", "cv"))
    gw, gmu = res.weights.cpu().numpy(), res.means.cpu().numpy()
    assert np.max(np.abs(gw - w) / np.maximum(w, 1e-6)) <= 1e-3
    assert np.max(np.abs(gmu - mu)) <= 1e-3 * np.max(np.abs(mu))


@pytest.mark.parametrize("cov", ["spherical", "diag", "tied", "full"])
def test_gaussian_mixture_class(torch_cuda, cov):
    """The scikit-learn style class: from a given init it holds exactly what
    fit() returns for that init (the same library calls), its state has the
    scikit-learn shapes, and predict_proba_topm agrees with the oracle's
    top-m on the rows whose decisions have a margin above 1e-6."""
    from soft_clustering_em_amd import estimator as est
    torch = torch_cuda
    N, D, K, m, thr = 4000, 8, 12, 4, 0.1
    rng = np.random.default_rng(7)
    X, w, mu, cv = _theta(rng, cov, N, D, K)
    if cov == "spherical":
        cv = np.full(K, float(X.var(axis=0).mean()), dtype=np.float32)
    tX = torch.from_numpy(X).cuda()
    gm = est.GaussianMixture(K, covariance_type=cov, max_iter=5, tol=0.0, weights_init=w, means_init=mu,
                             covariances_init=cv).fit(tX)
    init = tuple(torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (w, mu, cv))
    ref = est.fit(tX, K, cov, n_iter=5, tol=0.0, init=init)
    shapes = {"spherical": (K,), "diag": (K, D), "tied": (D, D), "full": (K, D, D)}
    assert tuple(gm.covariances_.shape) == shapes[cov]
    assert tuple(gm.means_.shape) == (K, D) and tuple(gm.weights_.shape) == (K,)
    assert torch.equal(gm.means_, ref.means) and torch.equal(gm.covariances_, ref.covars)
    assert gm.n_iter_ == 5 and len(gm.lower_bound_history_) == 5
    h = np.asarray(gm.lower_bound_history_)
    assert (np.diff(h) >= -1e-6 * np.abs(h[1:])).all(), h
    assert abs(gm.lower_bound_ - gm.score(tX)) <= 1e-9 * abs(gm.lower_bound_)
    idx, resp, cnt = gm.predict_proba_topm(tX, m=m, threshold=thr)
    th = tuple(t.cpu().numpy().astype(np.float64) for t in (gm.weights_, gm.means_, gm.covariances_))
    o_idx, o_resp, o_cnt, _, margin = oracle.topm(cov, X, *th, m, float(np.float32(thr)))
    ok = margin > 1e-6
    print(f"{cov}: topm rows checked {ok.sum()}/{N}, LL {h[0]:.4f} -> {h[-1]:.4f}", flush=True)
    assert ok.sum() > 0.9 * N
    assert np.array_equal(idx.cpu().numpy()[ok], o_idx[ok]) and np.array_equal(cnt.cpu().numpy()[ok], o_cnt[ok])
    assert np.max(np.abs(resp.cpu().numpy()[ok] - o_resp[ok])) <= 1e-4
    assert np.array_equal(gm.predict(tX).cpu().numpy()[ok], o_idx[ok, 0])


@pytest.mark.parametrize("cov", ["spherical", "diag"])
def test_gaussian_mixture_topk_mode_follows_the_oracle(torch_cuda, cov):
    """GaussianMixture(topk=k) runs approximate top-k EM steps: from a given
    init, two steps match the oracle's top-k steps (the second one from the
    oracle's own first-step parameters rounded to float32)."""
    from soft_clustering_em_amd.estimator import GaussianMixture
    torch = torch_cuda
    rng = np.random.default_rng(31)
    X, w, mu, cv = _theta(rng, cov, 3000, 10, 20)
    gm = GaussianMixture(20, covariance_type=cov, max_iter=2, tol=0.0, weights_init=w, means_init=mu,
                         covariances_init=cv, topk=3).fit(torch.from_numpy(X).cuda())
    th = (w.astype(np.float64), mu.astype(np.float64), cv.astype(np.float64))
    lls = []
    for _ in range(2):
        out = oracle.topk_fit_step(cov, X.astype(np.float64), *th, 3)
        lls.append(out["mean_ll"][0])
        th = tuple(out[k].astype(np.float32).astype(np.float64) for k in ("w", "mu", "cv"))
    assert np.allclose(gm.lower_bound_history_, lls, rtol=1e-6)
    gmu = gm.means_.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(gmu - th[1])) <= 1e-4 * max(1.0, np.max(np.abs(th[1])))
    assert abs(float(gm.weights_.double().sum().item()) - 1.0) < 1e-5


def test_kernel_density_class(torch_cuda):
    from soft_clustering_em_amd.estimator import KernelDensity
    torch = torch_cuda
    rng = np.random.default_rng(32)
    X = rng.normal(size=(700, 12)).astype(np.float32) * 2.0
    Y = rng.normal(size=(333, 12)).astype(np.float32) * 2.0
    kd = KernelDensity(bandwidth=0.9).fit(torch.from_numpy(X).cuda())
    got = kd.score_samples(torch.from_numpy(Y).cuda()).cpu().numpy().astype(np.float64)
    ref = oracle.kde_score(Y, X, 0.9)
    assert np.all(np.abs(got - ref) <= 1e-4 * np.maximum(1.0, np.abs(ref)))
    assert abs(kd.score(torch.from_numpy(Y).cuda()) - ref.sum()) <= 1e-4 * abs(ref.sum())
    with pytest.raises(ValueError):
        KernelDensity(bandwidth=0.0)
