"""gmm_fit: n_iter EM iterations in one call equal n_iter gmm_fit_step calls
bit for bit (parameters, per-iteration mean log-likelihoods, component
flags), for every covariance type, batched problems, collapsing components
and the large-K path.  gmm_fit_step itself is compared with the float64
oracle step by step in tests/test_gpu_parity.py and test_gpu_largek.py."""
import numpy as np
import pytest

from soft_clustering_em_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import soft_clustering_em_amd._abi as abi
    abi.lib()  # fails loudly if libgmm.so was not built
    return torch


def _clone(torch, wl):
    return tuple(torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (wl.w0, wl.mu0, wl.cv0))


def _x(torch, wl):
    if wl.xdtype == "bf16":
        return torch.from_numpy(wl.X.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(wl.X).cuda()


CASES = [
    ("spherical small", lambda: synth.spherical_small(N=10_000)),
    ("diag", lambda: synth.diag_large(N=60_000)),
    ("diag batched", lambda: synth.diag_batched(B=4, N=20_000)),
    ("full", lambda: synth.full_large(N=50_000)),
    ("ivf bf16 large-K", lambda: synth.ivf_bf16(N=40_000)),
]


@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("n_iter", [1, 5])
def test_fit_equals_repeated_fit_steps(torch_cuda, name, make, n_iter):
    import soft_clustering_em_amd as g
    torch = torch_cuda
    wl = make()
    X = _x(torch, wl)
    a = _clone(torch, wl)
    b = _clone(torch, wl)
    ws = torch.empty(g.gmm_workspace_bytes(X, wl.K, wl.cov), dtype=torch.uint8, device="cuda")
    mll_a = torch.zeros((n_iter, wl.B), dtype=torch.float64, device="cuda")
    cs_a = torch.full((wl.B, wl.K), -1, dtype=torch.int32, device="cuda")
    g.gmm_fit(X, *a, wl.cov, n_iter, reg_covar=wl.eps, mean_loglik=mll_a, comp_status=cs_a, ws=ws)
    mll_b = torch.zeros((n_iter, wl.B), dtype=torch.float64, device="cuda")
    cs_b = torch.full((wl.B, wl.K), -1, dtype=torch.int32, device="cuda")
    for t in range(n_iter):
        g.gmm_fit_step(X, *b, wl.cov, reg_covar=wl.eps, mean_loglik=mll_b[t], comp_status=cs_b, ws=ws)
    torch.cuda.synchronize()
    for ta, tb, what in zip(a, b, ("w", "mu", "cv")):
        assert torch.equal(ta, tb), (name, what, float((ta - tb).abs().max()))
    assert torch.equal(mll_a, mll_b), (name, mll_a, mll_b)
    assert torch.equal(cs_a, cs_b), name


def test_fit_tied_and_collapse(torch_cuda):
    """Tied components (their M-step is not fused: every iteration launches
    its prologue) and a diagonal case whose components collapse onto single
    rows (flags, kept parameters) through one call."""
    import soft_clustering_em_amd as g
    torch = torch_cuda
    rng = np.random.default_rng(5)
    for cov, D, K in (("tied", 6, 5), ("diag", 16, 40)):
        N = 2000
        X = (3.0 * rng.standard_normal((1, N, D))).astype(np.float32)
        mu0 = X[:, rng.choice(N, K, replace=False)].copy()
        w0 = np.full((1, K), 1.0 / K, np.float32)
        cv0 = (np.tile(np.eye(D, dtype=np.float32), (1, 1, 1)) if cov == "tied"
               else np.full((1, K, D), 1e-3, np.float32))
        wl = synth.Workload(f"{cov}-fit", cov, X, "f32", w0, mu0, cv0, iters=6)
        Xt = _x(torch, wl)
        a = _clone(torch, wl)
        b = _clone(torch, wl)
        ws = torch.empty(g.gmm_workspace_bytes(Xt, K, cov), dtype=torch.uint8, device="cuda")
        mll_a = torch.zeros((6, 1), dtype=torch.float64, device="cuda")
        cs_a = torch.full((1, K), -1, dtype=torch.int32, device="cuda")
        g.gmm_fit(Xt, *a, cov, 6, reg_covar=1e-6, mean_loglik=mll_a, comp_status=cs_a, ws=ws)
        mll_b = torch.zeros((6, 1), dtype=torch.float64, device="cuda")
        cs_b = torch.full((1, K), -1, dtype=torch.int32, device="cuda")
        for t in range(6):
            g.gmm_fit_step(Xt, *b, cov, reg_covar=1e-6, mean_loglik=mll_b[t], comp_status=cs_b, ws=ws)
        torch.cuda.synchronize()
        for ta, tb in zip(a, b):
            assert torch.equal(ta, tb), cov
        assert torch.equal(mll_a, mll_b) and torch.equal(cs_a, cs_b), cov


def test_fit_rejects_bad_arguments(torch_cuda):
    import soft_clustering_em_amd as g
    from soft_clustering_em_amd._abi import GmmError
    torch = torch_cuda
    wl = synth.spherical_small(N=1000)
    X = _x(torch, wl)
    w, mu, cv = _clone(torch, wl)
    with pytest.raises(GmmError):
        g.gmm_fit(X, w, mu, cv, wl.cov, 0)
    with pytest.raises(ValueError):
        g.gmm_fit(X, w, mu, cv, wl.cov, 4, mean_loglik=torch.zeros((3, 1), dtype=torch.float64, device="cuda"))
