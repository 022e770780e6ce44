"""Components in blocks: spherical and diagonal problems over float32-path rows
(float32, or 16-bit rows decoded to float32) with more components than one
workgroup holds (K above 256; above 128 for diagonal components at D = 128).
The fused kernel then runs per (problem, block of components): a pass that
writes each row's maximum and sum of 2^(l - max) over the block, a row
combine into the row's log-sum-exp and log-likelihood, and a pass that forms
the responsibilities against that log-sum-exp and adds the block's statistics
to the problem's partials.  One EM step from identical float32 parameters
against the float64 oracle, with the float32 bar of 1e-4 (2e-2 for 16-bit
rows), as for every other float32 workload; gmm_fit equal bit for bit to
repeated gmm_fit_step calls; statistics accumulated over row chunks."""
import numpy as np
import pytest

import oracle
from parity import TOL_F32, TOL_LOWP, oracle_trajectory, param_errors, to_np
from soft_clustering_em_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import soft_clustering_em_amd._abi as abi
    abi.lib()  # fails loudly if libgmm.so was not built
    return torch


def blobs(rng, B, N, D, K, spread=3.0):
    """K blobs per problem; each component starts at a row of its own blob
    (a random row where the blob drew none), so that no two components start
    in one blob and squeeze each other onto single rows in the first step --
    where the fused kernel's float32 logits, with or without blocks, bound the
    variance of such a component to about 1e-4 (the limit is measured and
    described with the design notes)."""
    X = np.empty((B, N, D), np.float32)
    mu0 = np.empty((B, K, D), np.float32)
    for b in range(B):
        centers = spread * rng.standard_normal((K, D))
        lab = rng.integers(0, K, N)
        X[b] = (centers[lab] + rng.uniform(0.5, 1.5, (N, 1)) * rng.standard_normal((N, D))).astype(np.float32)
        first = np.full(K, -1)
        rows = np.arange(N)[::-1]
        first[lab[rows]] = rows  # the first row of each blob
        none = first < 0
        first[none] = rng.choice(N, int(none.sum()))
        mu0[b] = X[b][first]
    return X, mu0


def workload(cov, B, N, D, K, seed):
    rng = np.random.default_rng(seed)
    X, mu0 = blobs(rng, B, N, D, K)
    w0 = np.full((B, K), 1.0 / K, np.float32)
    cv0 = np.ones((B, K), np.float32) if cov == "spherical" else np.ones((B, K, D), np.float32)
    return synth.Workload(f"{cov}-{B}x{N}x{D}-K{K}", cov, X, "f32", w0, mu0, cv0, iters=2)


def fit_step(torch, X, theta, cov, B, K, eps=1e-6):
    import soft_clustering_em_amd as g
    w, mu, cv = (torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in theta)
    mll = torch.zeros(B, dtype=torch.float64, device="cuda")
    cs = torch.full((B, K), -1, dtype=torch.int32, device="cuda")
    g.gmm_fit_step(X, w, mu, cv, cov, reg_covar=eps, mean_loglik=mll, comp_status=cs)
    torch.cuda.synchronize()
    return (to_np(w), to_np(mu), to_np(cv)), to_np(mll), cs.cpu().numpy()


def check(torch, wl, th, out, X, label, tol=TOL_F32):
    (wg, mg, cg), mll, cs = fit_step(torch, X, th, wl.cov, wl.B, wl.K, wl.eps)
    e = param_errors(wl.cov, wl.B, wl.K, wl.D, (wg, mg, cg), (out["w"], out["mu"], out["cv"]), out["stats"]["nk"])
    e_ll = float(np.max(np.abs(mll - out["mean_ll"]) / np.abs(out["mean_ll"])))
    print(f"{label} mu={e['mu']:.2e} cv={e['cv']:.2e} w={e['w']:.2e} ll={e_ll:.2e} live={e['live']}", flush=True)
    assert e["mu"] <= tol and e["cv"] <= tol and e["w"] <= tol and e_ll <= tol, (label, e, e_ll)
    assert e["w_abs_small"] <= 1e-10
    assert (cs >= 0).all()


BLOCKED = [
    # cov, B, N, D, K: blocks of 256 components (128 for diagonal at D = 128)
    ("spherical", 1, 20_000, 16, 300),    # two blocks, the second mostly padding
    ("diag", 1, 20_011, 32, 520),         # three blocks, ragged rows
    ("diag", 1, 16_000, 128, 200),        # D = 128 diagonal: blocks of 128
    ("spherical", 2, 6_000, 8, 700),      # several problems, three blocks each
    ("diag", 1, 30_000, 64, 1024),        # four full blocks
    ("spherical", 1, 20_000, 3, 2049),    # nine blocks, the last with one component
]


@pytest.mark.parametrize("cov,B,N,D,K", BLOCKED)
def test_blocked_components_two_steps(torch_cuda, cov, B, N, D, K):
    wl = workload(cov, B, N, D, K, seed=N + D + K)
    thetas, outs = oracle_trajectory(wl, 2)
    X = torch_cuda.from_numpy(wl.X).cuda()
    for t in range(2):
        check(torch_cuda, wl, thetas[t], outs[t], X, f"{wl.name} t={t}")


def test_blocked_rows_past_one_chunk(torch_cuda):
    """More rows than one chunk of the blocked E-step (2^20): the second chunk's
    statistics and log-likelihood are added to the first's."""
    wl = workload("spherical", 1, (1 << 20) + 4_999, 8, 300, seed=7)
    thetas, outs = oracle_trajectory(wl, 1)
    check(torch_cuda, wl, thetas[0], outs[0], torch_cuda.from_numpy(wl.X).cuda(), "two chunks")


def test_blocked_fit_equals_repeated_steps_and_is_deterministic(torch_cuda):
    import soft_clustering_em_amd as g
    torch = torch_cuda
    wl = workload("diag", 1, 30_000, 32, 600, seed=3)
    X = torch.from_numpy(wl.X).cuda()
    ws = torch.empty(g.gmm_workspace_bytes(X, wl.K, wl.cov), dtype=torch.uint8, device="cuda")
    runs = []
    for _ in range(2):
        a = tuple(torch.from_numpy(np.ascontiguousarray(t)).cuda() for t in (wl.w0, wl.mu0, wl.cv0))
        mll = torch.zeros((4, 1), dtype=torch.float64, device="cuda")
        g.gmm_fit(X, *a, wl.cov, 4, mean_loglik=mll, ws=ws)
        runs.append((a, mll))
    b = tuple(torch.from_numpy(np.ascontiguousarray(t)).cuda() for t in (wl.w0, wl.mu0, wl.cv0))
    mll_b = torch.zeros((4, 1), dtype=torch.float64, device="cuda")
    for t in range(4):
        g.gmm_fit_step(X, *b, wl.cov, mean_loglik=mll_b[t], ws=ws)
    torch.cuda.synchronize()
    for (a, mll) in runs:
        for ta, tb in zip(a, b):
            assert torch.equal(ta, tb)
        assert torch.equal(mll, mll_b)
    ll = mll_b.cpu().numpy()[:, 0]
    assert np.all(np.diff(ll) >= -1e-9 * np.abs(ll[:-1])), ll  # EM never lowers the likelihood


def test_blocked_chunked_statistics(torch_cuda):
    """gmm_estep_stats over row chunks with accumulate, then one M-step, equal
    the oracle's statistics and step."""
    import soft_clustering_em_amd as g
    torch = torch_cuda
    wl = workload("diag", 1, 12_000, 16, 400, seed=11)
    X = torch.from_numpy(wl.X).cuda()
    w, mu, cv = (torch.from_numpy(a.copy()).cuda() for a in (wl.w0, wl.mu0, wl.cv0))
    st = g.new_stats(1, wl.K, wl.D, "diag", "cuda")
    bounds = [0, 5_000, 5_001, 12_000]
    for i in range(len(bounds) - 1):
        g.gmm_estep_stats(X[:, bounds[i]:bounds[i + 1]], w, mu, cv, "diag", st, accumulate=i > 0)
    ref = oracle.estep("diag", wl.X[0], wl.w0[0], wl.mu0[0], wl.cv0[0])
    nk = to_np(st["nk"])[0]
    np.testing.assert_allclose(nk.sum(), wl.N, rtol=1e-6)
    live = ref["nk"][0] >= 1
    np.testing.assert_allclose(nk[live], ref["nk"][0][live], rtol=1e-4)
    assert abs(to_np(st["loglik"])[0] - ref["ll"][0]) <= 1e-5 * abs(ref["ll"][0])
    g.gmm_mstep(st, wl.N, w, mu, cv, "diag", reg_covar=wl.eps)
    torch.cuda.synchronize()
    out = oracle.fit_step("diag", wl.X[0], wl.w0[0], wl.mu0[0], wl.cv0[0], eps=wl.eps)
    e = param_errors("diag", 1, wl.K, wl.D, (to_np(w), to_np(mu), to_np(cv)),
                     (out["w"], out["mu"], out["cv"]), out["stats"]["nk"])
    assert e["mu"] <= TOL_F32 and e["cv"] <= TOL_F32 and e["w"] <= TOL_F32, e


@pytest.mark.parametrize("kind,cov,B,K", [("bf16", "diag", 1, 300), ("f16", "spherical", 1, 600),
                                          ("bf16", "spherical", 2, 400)])
def test_blocked_16bit_rows(torch_cuda, kind, cov, B, K):
    """16-bit rows (decoded exactly to float32 as tiles are staged) with blocks:
    the oracle reads the same 16-bit values; the 16-bit bar is 2e-2."""
    torch = torch_cuda
    rng = np.random.default_rng(K + B)
    N, D = 9_000, 24
    Xf, _ = blobs(rng, B, N, D, K)
    if kind == "f16":
        h = Xf.astype(np.float16)
        X = torch.from_numpy(h).cuda()
        Xo = [(h[b].view(np.uint16), "f16") for b in range(B)]
        X64 = h.astype(np.float64)
    else:
        bits = synth.f32_to_bf16_bits(Xf)
        X = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
        Xo = [(bits[b], "bf16") for b in range(B)]
        X64 = synth.bf16_bits_to_f32(bits).astype(np.float64)
    w = np.full((B, K), 1.0 / K, np.float32)
    mu = np.stack([X64[b][rng.choice(N, K, replace=False)] for b in range(B)]).astype(np.float32)
    cv = np.ones((B, K), np.float32) if cov == "spherical" else rng.uniform(0.5, 2.0, (B, K, D)).astype(np.float32)
    got, mll, _ = fit_step(torch, X, (w, mu, cv), cov, B, K)
    for b in range(B):
        o = oracle.fit_step(cov, Xo[b], w[b].astype(np.float64), mu[b].astype(np.float64), cv[b].astype(np.float64))
        e = param_errors(cov, 1, K, D, tuple(a[b] for a in got), (o["w"], o["mu"], o["cv"]), o["stats"]["nk"])
        e_ll = abs(float(mll[b]) - o["mean_ll"][0]) / abs(o["mean_ll"][0])
        print(f"{kind} {cov} B={B} K={K} b={b}: mu={e['mu']:.1e} cv={e['cv']:.1e} w={e['w']:.1e} ll={e_ll:.1e}",
              flush=True)
        assert max(e["mu"], e["cv"], e["w"], e_ll) <= TOL_LOWP, (b, e, e_ll)


def test_blocked_window_limit(torch_cuda):
    """Above 8192 spherical / diagonal components (and for full and tied
    components above one workgroup) the call is refused before any launch."""
    import soft_clustering_em_amd as g
    from soft_clustering_em_amd import _abi
    torch = torch_cuda
    X = torch.zeros(100, 4, device="cuda")
    for cov, K in (("diag", 8193), ("full", 257)):
        w = torch.full((1, K), 1.0 / K, device="cuda")
        mu = torch.zeros(1, K, 4, device="cuda")
        cv = torch.ones(*g.cov_shape(cov, 1, K, 4), device="cuda")
        with pytest.raises(g.GmmError) as ei:
            g.gmm_fit_step(X, w, mu, cv, cov)
        assert ei.value.status == _abi.GMM_ERR_UNSUPPORTED


@pytest.mark.parametrize("K", [64, 300])
def test_wave_without_live_components_and_low_scores(torch_cuda, K):
    """Components 32..255 carry weight 0, so whole waves hold no live
    component (K = 300 adds the padding waves of its last block), and every
    row's best log2 score lies below -128 (D = 64, unit variances, rows 1.5
    sigma from their mean: about -190).  A wave with no live component once
    took 2^(0 - M) = +inf as its share of such a row (NaN statistics); the step
    must stay finite and match the oracle, the empty components flagged and
    kept at weight 0."""
    rng = np.random.default_rng(K)
    N, D = 6_000, 64
    live = np.r_[np.arange(32), np.arange(256, K)]
    mu = (3.0 * rng.standard_normal((1, K, D))).astype(np.float32)
    lab = rng.choice(live, N)
    X = (mu[0][lab] + 1.5 * rng.standard_normal((N, D)))[None].astype(np.float32)
    w = np.zeros((1, K), np.float32)
    w[0, live] = 1.0 / len(live)
    cv = np.ones((1, K, D), np.float32)
    o = oracle.fit_step("diag", X[0], w[0].astype(np.float64), mu[0].astype(np.float64), cv[0].astype(np.float64))
    _, _, lse = oracle.responsibilities("diag", X[0], w[0].astype(np.float64), mu[0].astype(np.float64),
                                        cv[0].astype(np.float64))
    assert np.max(lse) < -128 * np.log(2), "every row's best score below -128 in log2 units"
    (wg, mg, cg), mll, cs = fit_step(torch_cuda, torch_cuda.from_numpy(X).cuda(), (w, mu, cv), "diag", 1, K)
    assert np.isfinite(wg).all() and np.isfinite(mg).all() and np.isfinite(cg).all() and np.isfinite(mll).all()
    e = param_errors("diag", 1, K, D, (wg, mg, cg), (o["w"], o["mu"], o["cv"]), o["stats"]["nk"])
    e_ll = abs(float(mll[0]) - o["mean_ll"][0]) / abs(o["mean_ll"][0])
    print(f"waves without live components, K={K}: mu={e['mu']:.1e} cv={e['cv']:.1e} w={e['w']:.1e} "
          f"ll={e_ll:.1e}", flush=True)
    assert max(e["mu"], e["cv"], e["w"], e_ll) <= TOL_F32, (e, e_ll)
    dead = w[0] == 0
    assert (wg.reshape(K)[dead] == 0).all() and (cs.reshape(K)[dead] == 1).all()
