"""Parity of gmm_topk_fit_step (approximate top-k EM, the approx_top_k mode of
the GMMXX README: each row keeps its k best log-scores and normalises over
them; k >= K is exact EM) against the float64 oracle (oracle.topk_fit_step,
pinned by its k >= K, k = 1 and common-kept-set special cases), one step from
identical float32 parameters.  The kept sets are decided on float64 scores on
both sides and the statistics are float64 sums of float32 responsibilities,
so the float32 bar of 1e-4 holds for bf16 rows too."""
import numpy as np
import pytest

import oracle
from parity import TOL_F32, param_errors, to_np
from soft_clustering_em_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import soft_clustering_em_amd._abi as abi
    abi.lib()
    return torch


def theta(rng, cov, B, K, D, X):
    w = np.stack([rng.dirichlet(np.full(K, 3.0)) for _ in range(B)]).astype(np.float32)
    mu = np.stack([X[b][rng.choice(X.shape[1], K, replace=False)] for b in range(B)]).astype(np.float32)
    if cov == "spherical":
        cv = rng.uniform(0.5, 2.0, size=(B, K)).astype(np.float32)
    else:
        cv = rng.uniform(0.5, 2.0, size=(B, K, X.shape[2])).astype(np.float32)
    return w, mu, cv


def gpu_step(torch, Xd, th, cov, topk):
    import soft_clustering_em_amd as g
    w, mu, cv = (torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in th)
    B = w.shape[0]
    mll = torch.zeros(B, dtype=torch.float64, device="cuda")
    cs = torch.full(w.shape, -1, dtype=torch.int32, device="cuda")
    g.gmm_topk_fit_step(Xd, w, mu, cv, cov, topk, mean_loglik=mll, comp_status=cs)
    torch.cuda.synchronize()
    return (to_np(w), to_np(mu), to_np(cv)), to_np(mll), cs.cpu().numpy()


def check(label, cov, X64, th, got, mll, topk):
    B, K = th[0].shape
    D = X64.shape[2]
    for b in range(B):
        ref = oracle.topk_fit_step(cov, X64[b], *(a[b].astype(np.float64) for a in th), topk)
        e = param_errors(cov, 1, K, D, tuple(a[b] for a in got), (ref["w"], ref["mu"], ref["cv"]), ref["stats"]["nk"])
        e_ll = abs(mll[b] - ref["mean_ll"][0]) / abs(ref["mean_ll"][0])
        print(f"{label} b={b}: mu={e['mu']:.2e} cv={e['cv']:.2e} w={e['w']:.2e} ll={e_ll:.2e}", flush=True)
        assert e["mu"] <= TOL_F32 and e["cv"] <= TOL_F32 and e["w"] <= TOL_F32 and e_ll <= 1e-6, (label, b, e, e_ll)


@pytest.mark.parametrize("cov", ["spherical", "diag"])
@pytest.mark.parametrize("B,N,D,K,topk", [(1, 3001, 12, 20, 3), (3, 2000, 7, 33, 1), (2, 1500, 16, 40, 16),
                                          (1, 4000, 10, 300, 4)])  # K > 256: the exact top-m kernel
def test_topk_step_float32(torch_cuda, cov, B, N, D, K, topk):
    torch = torch_cuda
    rng = np.random.default_rng(N + K + topk)
    X = (rng.normal(size=(B, N, D)) + 3.0 * rng.integers(0, 6, size=(B, N, 1)) * rng.normal(size=(B, 1, D))).astype(np.float32)
    th = theta(rng, cov, B, K, D, X)
    got, mll, cs = gpu_step(torch, torch.from_numpy(X).cuda(), th, cov, topk)
    check(f"{cov} B={B} N={N} D={D} K={K} k={topk}", cov, X.astype(np.float64), th, got, mll, topk)
    assert (cs >= 0).all()


@pytest.mark.parametrize("cov", ["spherical", "diag"])
def test_topk_with_every_component_is_the_exact_step(torch_cuda, cov):
    """k >= K: the GPU top-k step equals the oracle's exact EM step and the GPU
    exact step (the page: values >= K resolve to exact EM)."""
    import soft_clustering_em_amd as g
    torch = torch_cuda
    rng = np.random.default_rng(41)
    B, N, D, K = 1, 4000, 10, 12
    X = rng.normal(size=(B, N, D)).astype(np.float32) * 2.0
    th = theta(rng, cov, B, K, D, X)
    Xd = torch.from_numpy(X).cuda()
    got, mll, _ = gpu_step(torch, Xd, th, cov, 16)
    ref = oracle.fit_step(cov, X[0].astype(np.float64), *(a[0].astype(np.float64) for a in th))
    e = param_errors(cov, 1, K, D, got, (ref["w"], ref["mu"], ref["cv"]), ref["stats"]["nk"])
    assert e["mu"] <= TOL_F32 and e["cv"] <= TOL_F32 and e["w"] <= TOL_F32, e
    assert abs(mll[0] - ref["mean_ll"][0]) <= 1e-6 * abs(ref["mean_ll"][0])
    w, mu, cv = (torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in th)
    m2 = torch.zeros(B, dtype=torch.float64, device="cuda")
    g.gmm_fit_step(Xd, w, mu, cv, cov, mean_loglik=m2)
    e = param_errors(cov, B, K, D, got, (to_np(w), to_np(mu), to_np(cv)), np.full((B, K), 10.0))
    assert e["mu"] <= 1e-5 and e["cv"] <= 1e-5 and e["w"] <= 1e-5, e
    assert abs(mll[0] - float(m2[0])) <= 1e-6 * abs(float(m2[0]))


@pytest.mark.parametrize("cov", ["spherical", "diag"])
def test_topk_step_float32_far_tail(torch_cuda, cov):
    """256 well-separated clusters in 64 dimensions, components started at
    data rows, k = 4: the 2nd-4th kept components of most rows carry
    responsibilities far below 2^-20, and for components with few rows of
    their own those tiny weights make much of the scatter (dropping them
    would change variances by up to 0.5 relative here)."""
    torch = torch_cuda
    N, D, K, topk = 5003, 64, 256, 4
    rng = np.random.default_rng(N + topk)
    centers = 3.0 * rng.standard_normal((K, D))
    X = (centers[rng.integers(0, K, N)] + rng.standard_normal((N, D))).astype(np.float32)[None]
    th = theta(rng, cov, 1, K, D, X)
    got, mll, cs = gpu_step(torch, torch.from_numpy(X).cuda(), th, cov, topk)
    check(f"far tail {cov}", cov, X.astype(np.float64), th, got, mll, topk)


@pytest.mark.parametrize("cov", ["spherical", "diag"])
def test_topk_keeps_far_rows_of_a_narrow_component(torch_cuda, cov):
    """k = 2 of K = 3, the third component far away (every row keeps 0 and 1):
    component 1 is narrow, so most rows give it a responsibility far below
    2^-20 that is still kept and still carries its scatter.  Checked against
    the oracle (which the pins tie to exact EM of the two-component
    sub-mixture here)."""
    torch = torch_cuda
    rng = np.random.default_rng(35)
    D, N = 2, 6000
    X = rng.normal(size=(N, D))
    X[:2] = [[0.5, 0.5], [0.5 + 1e-3, 0.5]]
    X = X.astype(np.float32)
    w = np.array([[0.5, 0.3, 0.2]], np.float32)
    mu = np.array([[[0.0, 0.0], [0.5 + 5e-4, 0.5], [400.0, -400.0]]], np.float32)
    cv = (np.array([[1.0, 1e-3, 1.0]]) if cov == "spherical" else
          np.array([[[1.0, 1.2], [1e-3, 2e-3], [1.0, 1.0]]])).astype(np.float32)
    got, mll, cs = gpu_step(torch, torch.from_numpy(X[None]).cuda(), (w, mu, cv), cov, 2)
    check(f"narrow {cov}", cov, X[None].astype(np.float64), (w, mu, cv), got, mll, 2)


@pytest.mark.parametrize("N,D,K,topk", [(5003, 128, 512, 4), (3000, 100, 300, 2), (4099, 128, 700, 16),
                                        (2000, 128, 600, 1)])
def test_topk_step_bf16_rows(torch_cuda, N, D, K, topk):
    """bf16 rows take the large-K top-m in its top-k mode (spherical, any K);
    D = 128 forms the per-row top-k threshold, D = 100 rescores every
    component of a row."""
    torch = torch_cuda
    rng = np.random.default_rng(N + topk)
    centers = 3.0 * rng.standard_normal((K, D))
    Xf = (centers[rng.integers(0, K, N)] + rng.standard_normal((N, D))).astype(np.float32)
    bits = synth.f32_to_bf16_bits(Xf)
    X64 = synth.bf16_bits_to_f32(bits).astype(np.float64)[None]
    th = theta(rng, "spherical", 1, K, D, X64.astype(np.float32))
    Xd = torch.from_numpy(np.ascontiguousarray(bits[None]).view(np.int16)).cuda().view(torch.bfloat16)
    got, mll, cs = gpu_step(torch, Xd, th, "spherical", topk)
    check(f"bf16 N={N} D={D} K={K} k={topk}", "spherical", X64, th, got, mll, topk)


def test_topk_step_is_deterministic(torch_cuda):
    torch = torch_cuda
    rng = np.random.default_rng(42)
    X = rng.normal(size=(1, 20000, 32)).astype(np.float32)
    th = theta(rng, "diag", 1, 64, 32, X)
    Xd = torch.from_numpy(X).cuda()
    a = gpu_step(torch, Xd, th, "diag", 4)
    b = gpu_step(torch, Xd, th, "diag", 4)
    for u, v in zip(a[0], b[0]):
        assert np.array_equal(u, v)
    assert np.array_equal(a[1], b[1])


def test_topk_step_bf16_collapsed_component(torch_cuda):
    """bf16 rows, K = 512: one component collapsed (variance 1e-4) onto a
    tight group of rows, k = 4 -- far rows keep it among their top 4 with
    tiny responsibilities that carry much of its scatter."""
    torch = torch_cuda
    rng = np.random.default_rng(77)
    N, D, K = 6000, 128, 512
    centers = rng.standard_normal((K, D)) / np.sqrt(D)
    Xf = (centers[rng.integers(0, K, N)] + 0.05 * rng.standard_normal((N, D))).astype(np.float32)
    Xf[:40] = centers[0] + 0.01 * rng.standard_normal((40, D))
    bits = synth.f32_to_bf16_bits(Xf)
    X64 = synth.bf16_bits_to_f32(bits).astype(np.float64)[None]
    w = np.full((1, K), 1.0 / K, np.float32)
    mu = centers[None].astype(np.float32)
    cv = np.full((1, K), 0.05 ** 2, np.float32)
    cv[0, 0] = 1e-4
    Xd = torch.from_numpy(np.ascontiguousarray(bits[None]).view(np.int16)).cuda().view(torch.bfloat16)
    got, mll, cs = gpu_step(torch, Xd, (w, mu, cv), "spherical", 4)
    check("bf16 collapsed K=512 k=4", "spherical", X64, (w, mu, cv), got, mll, 4)


def test_topk_step_full_size_properties(torch_cuda):
    """1M rows x D = 64, K = 256 (the diagonal benchmark workload), k = 4: the
    weights sum to 1, no component fails, and per row the log sum over the kept
    set lies between log p(x) - log(K / k) (the k largest of K terms hold at
    least k / K of the mass) and log p(x), so the step's mean LL lies in that
    range of the exact step's."""
    import soft_clustering_em_amd as g
    torch = torch_cuda
    wl = synth.diag_large()
    X = torch.from_numpy(wl.X).cuda()
    th = tuple(np.ascontiguousarray(a) for a in (wl.w0, wl.mu0, wl.cv0))
    got, mll, cs = gpu_step(torch, X, th, "diag", 4)
    w, mu, cv = (torch.from_numpy(a).cuda() for a in th)
    m2 = torch.zeros(1, dtype=torch.float64, device="cuda")
    g.gmm_fit_step(X, w, mu, cv, "diag", mean_loglik=m2)
    exact = float(m2[0])
    print(f"full size: top-k mean LL {mll[0]:.6f}, exact {exact:.6f}", flush=True)
    assert (cs >= 0).all()
    assert abs(float(got[0].astype(np.float64).sum()) - 1.0) < 1e-5
    assert exact - np.log(256 / 4) - 1e-6 <= mll[0] <= exact + 1e-6 * abs(exact)
    assert np.isfinite(got[1]).all() and (got[2] > 0).all()
