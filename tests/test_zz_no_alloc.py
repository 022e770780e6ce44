"""gmm_fit_step_noalloc (the fit step whose scratch is the library's static
device array, for callers that cannot allocate) against gmm_fit_step (the
same step with a caller workspace), through the C ABI: two calls in a row,
the second on a smaller input, each compared with the workspace entry point
on identical parameters to the float32 bar (1e-4; the two share kernels and
workspace layout, so they are expected to agree bit for bit)."""
import numpy as np
import pytest

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


def both(torch, X, th, cov):
    import soft_clustering_em_amd as g
    out = []
    for fn in ("gmm_fit_step", "gmm_fit_step_noalloc"):
        w, mu, cv = (torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in th)
        mll = torch.zeros(w.shape[0], dtype=torch.float64, device="cuda")
        cs = torch.full(w.shape, -1, dtype=torch.int32, device="cuda")
        getattr(g, fn)(X, w, mu, cv, cov, mean_loglik=mll, comp_status=cs)
        torch.cuda.synchronize()
        out.append(((to_np(w), to_np(mu), to_np(cv)), to_np(mll), cs.cpu().numpy()))
    return out


@pytest.mark.parametrize("cov", ["spherical", "diag", "full"])
def test_noalloc_matches_the_workspace_entry_point(torch_cuda, cov):
    torch = torch_cuda
    rng = np.random.default_rng(5)
    B, K, D = 2, 16, 8
    X = (rng.normal(size=(B, 10000, D)) * 2.0 + 4.0 * rng.integers(0, 4, size=(B, 10000, 1))).astype(np.float32)
    for N in (10000, 3001):  # two calls in a row, the second smaller
        Xn = np.ascontiguousarray(X[:, :N])
        w = np.full((B, K), 1.0 / K, np.float32)
        mu = np.ascontiguousarray(Xn[:, :K])
        if cov == "spherical":
            cv = np.ones((B, K), np.float32)
        elif cov == "diag":
            cv = np.ones((B, K, D), np.float32)
        else:
            cv = np.broadcast_to(np.eye(D, dtype=np.float32), (B, K, D, D)).copy()
        (ref, ll_ref, cs_ref), (got, ll, cs) = both(torch, torch.from_numpy(Xn).cuda(), (w, mu, cv), cov)
        e = param_errors(cov, B, K, D, got, ref, np.full((B, K), 10.0))
        e_ll = float(np.max(np.abs(ll - ll_ref) / np.abs(ll_ref)))
        same = all(np.array_equal(a, b) for a, b in zip(got, ref)) and np.array_equal(ll, ll_ref)
        print(f"{cov} N={N}: mu={e['mu']:.1e} cv={e['cv']:.1e} w={e['w']:.1e} ll={e_ll:.1e} bitwise={same}", flush=True)
        assert e["mu"] <= TOL_F32 and e["cv"] <= TOL_F32 and e["w"] <= TOL_F32 and e_ll <= TOL_F32
        assert np.array_equal(cs, cs_ref)


def test_noalloc_bf16_large_k_rows(torch_cuda):
    """bf16 rows (the large-K path) streamed through the static array in
    shorter chunks: the same step as with a full workspace, to the bf16 bar."""
    torch = torch_cuda
    for N in (6000, 2500):
        wl = synth.ivf_bf16(N=N, K=512)
        X = torch.from_numpy(wl.X.view(np.int16)).cuda().view(torch.bfloat16)
        th = (wl.w0, wl.mu0, wl.cv0)
        (ref, ll_ref, _), (got, ll, _) = both(torch, X, th, "spherical")
        e = param_errors("spherical", 1, wl.K, wl.D, got, ref, np.full((1, wl.K), 10.0))
        e_ll = float(abs(ll[0] - ll_ref[0]) / abs(ll_ref[0]))
        print(f"bf16 N={N} K=512: mu={e['mu']:.1e} cv={e['cv']:.1e} w={e['w']:.1e} ll={e_ll:.1e}", flush=True)
        assert e["mu"] <= 2e-2 and e["cv"] <= 2e-2 and e["w"] <= 2e-2 and e_ll <= 2e-2
