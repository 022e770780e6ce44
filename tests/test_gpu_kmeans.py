"""Parity of gmm_kmeans_step (one k-means / Lloyd iteration) against the
float64 oracle (oracle.kmeans_step).

Labels are compared element by element on the rows whose two smallest
squared distances differ by more than 1e-9 of the row's scale (|x|^2 +
max |c|^2): below that, the float64 rounding of either side may decide.  The
updated centroids, counts and inertia are compared exactly where every label
is decided, else within the effect of the undecided rows.  Centroids are
float32 means of float64 sums: 1e-6 relative (float32 rows) or, for bf16
rows, the same bar (the rows are decoded exactly on both sides).
"""
import numpy as np
import pytest

import oracle
from soft_clustering_em_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import soft_clustering_em_amd._abi as abi
    abi.lib()
    return torch


def blobs(rng, N, D, K, spread=4.0):
    cen = spread * rng.standard_normal((K, D))
    lab = rng.integers(0, K, N)
    return (cen[lab] + rng.uniform(0.5, 1.5, (N, 1)) * rng.standard_normal((N, D))).astype(np.float32)


def decided(X64, C64, gap):
    scale = np.sum(X64 * X64, axis=1) + np.max(np.sum(C64 * C64, axis=1))
    return gap > 1e-9 * scale


def gpu_kmeans(torch, Xd, C):
    import soft_clustering_em_amd as g
    Cd = torch.from_numpy(np.ascontiguousarray(C, dtype=np.float32)).cuda()
    lab, cnt, inert = g.gmm_kmeans_step(Xd, Cd)
    torch.cuda.synchronize()
    return lab.cpu().numpy(), Cd.cpu().numpy(), cnt.cpu().numpy(), inert.cpu().numpy()


def compare(label, X64, C, o, g, rtol_c=1e-6):
    o_lab, gap, o_newC, o_cnt, o_in = o
    g_lab, g_newC, g_cnt, g_in = g
    ok = decided(X64, C.astype(np.float64), gap)
    bad = np.nonzero(ok & (g_lab != o_lab))[0]
    print(f"{label}: rows {len(o_lab)}, undecided {int((~ok).sum())}, label mismatches {bad.size}", flush=True)
    assert bad.size == 0, (label, bad[:5], g_lab[bad[:5]], o_lab[bad[:5]])
    if ok.all():
        assert np.array_equal(g_cnt, o_cnt), label
        np.testing.assert_allclose(g_newC, o_newC.astype(np.float32), rtol=rtol_c, atol=1e-6 * np.abs(o_newC).max())
        assert abs(g_in - o_in) <= 1e-9 * abs(o_in) + 1e-300, (label, g_in, o_in)
        empty = o_cnt == 0
        assert np.array_equal(g_newC[empty], C[empty].astype(np.float32)), label


@pytest.mark.parametrize("N,D,K", [(10_000, 8, 16), (5003, 7, 13), (4096, 64, 256), (2500, 128, 40),
                                   (777, 3, 1), (1, 16, 4), (65, 33, 64),
                                   (6_000, 24, 700)])  # K > 256: labels from the exact top-m kernel
def test_kmeans_step_float32_rows(torch_cuda, N, D, K):
    torch = torch_cuda
    rng = np.random.default_rng(N + 7 * D + K)
    X = blobs(rng, N, D, K)
    C = X[rng.choice(N, K, replace=N < K)].astype(np.float64)
    o = oracle.kmeans_step(X, C)
    g = gpu_kmeans(torch, torch.from_numpy(X).cuda(), C)
    compare(f"f32 {N}x{D} K={K}", X.astype(np.float64), C, o, (g[0][0], g[1], g[2][0], g[3][0]))


def test_kmeans_step_batched_problems(torch_cuda):
    """B = 3 problems in one call, each against its own centroids; a problem
    b equals the single-problem call on X_b."""
    torch = torch_cuda
    rng = np.random.default_rng(5)
    B, N, D, K = 3, 3001, 12, 20
    X = np.stack([blobs(rng, N, D, K) for _ in range(B)])
    C = np.stack([X[b][rng.choice(N, K, replace=False)] for b in range(B)]).astype(np.float64)
    g = gpu_kmeans(torch, torch.from_numpy(X).cuda(), C)
    for b in range(B):
        o = oracle.kmeans_step(X[b], C[b])
        compare(f"batched b={b}", X[b].astype(np.float64), C[b], o, (g[0][b], g[1][b], g[2][b], g[3][b]))
        s = gpu_kmeans(torch, torch.from_numpy(X[b]).cuda(), C[b])
        assert np.array_equal(s[0][0], g[0][b]) and np.array_equal(s[1], g[1][b])


@pytest.mark.parametrize("N,D,K", [(20_011, 128, 512), (5003, 100, 300), (3000, 8, 16)])
def test_kmeans_step_bf16_rows(torch_cuda, N, D, K):
    """bf16 rows take the large-K top-1 (any K)."""
    torch = torch_cuda
    rng = np.random.default_rng(N + K)
    bits = synth.f32_to_bf16_bits(blobs(rng, N, D, K))
    X64 = synth.bf16_bits_to_f32(bits).astype(np.float64)
    C = X64[rng.choice(N, K, replace=False)]
    o = oracle.kmeans_step((bits, "bf16"), C)
    Xd = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)
    g = gpu_kmeans(torch, Xd, C)
    compare(f"bf16 {N}x{D} K={K}", X64, C, o, (g[0][0], g[1], g[2][0], g[3][0]))


def test_kmeans_ivf_rows_sampled(torch_cuda):
    """The IVF workload's unit rows (bf16, D = 128) on 200,000 rows against
    K = 4096 centroids drawn from them: labels of 3,000 sampled rows against
    the oracle, counts add up to N, and the centroid of sampled clusters is
    the float64 mean of the rows the GPU labelled into it."""
    torch = torch_cuda
    wl = synth.ivf_bf16(N=200_000)
    bits = wl.X[0]
    rng = np.random.default_rng(3)
    X64 = synth.bf16_bits_to_f32(bits).astype(np.float64)
    C = wl.mu0[0].astype(np.float64)
    Xd = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)
    g_lab, g_newC, g_cnt, g_in = gpu_kmeans(torch, Xd, C)
    g_lab, g_cnt = g_lab[0], g_cnt[0]
    assert g_cnt.sum() == len(bits) and np.array_equal(np.bincount(g_lab, minlength=4096), g_cnt)
    pick = rng.choice(len(bits), 3000, replace=False)
    o_lab, gap, _, _, _ = oracle.kmeans_step(X64[pick], C)
    ok = decided(X64[pick], C, gap)
    print(f"ivf sampled rows: undecided {int((~ok).sum())} of 3000", flush=True)
    assert np.array_equal(g_lab[pick][ok], o_lab[ok])
    for k in rng.choice(4096, 50, replace=False):
        rows = X64[g_lab == k]
        want = rows.mean(axis=0) if len(rows) else C[k]
        np.testing.assert_allclose(g_newC[k], want.astype(np.float32), rtol=1e-6, atol=1e-7)


def test_kmeans_bf16_near_ties_across_slices(torch_cuda):
    """Rows near the midpoint of two centroids whose indices lie in different
    256-centroid slices (K = 4096, bf16 rows of 128): the best and second best
    distances nearly tie, so each row's label rests on the candidate band of
    the one-pass marking (the error bounds alone) and on the slice test of the
    rescoring.  Labels equal the oracle's on every row the float64 gap
    decides, and most rows are decided."""
    torch = torch_cuda
    rng = np.random.default_rng(41)
    K, D, N = 4096, 128, 3000
    C = rng.standard_normal((K, D)).astype(np.float32).astype(np.float64)
    a = rng.integers(0, K, N)
    b = (a + 256 * rng.integers(1, 16, N) + rng.integers(0, 256, N)) % K
    X = 0.5 * (C[a] + C[b]) + 1e-3 * rng.standard_normal((N, D))
    bits = synth.f32_to_bf16_bits(X.astype(np.float32))
    X64 = synth.bf16_bits_to_f32(bits).astype(np.float64)
    o = oracle.kmeans_step((bits, "bf16"), C)
    Xd = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)
    g = gpu_kmeans(torch, Xd, C)
    ok = decided(X64, C, o[1])
    assert ok.mean() > 0.9, ok.mean()
    assert set(np.unique(o[0][ok] // 256).tolist()) != {0}  # labels spread over the slices
    compare("bf16 near ties across slices", X64, C, o, (g[0][0], g[1], g[2][0], g[3][0]))


def test_kmeans_empty_cluster_and_no_rows(torch_cuda):
    """A centroid no row is nearest to keeps its bits and counts 0; with
    N = 0 every centroid is kept, counts are 0 and the inertia is 0."""
    torch = torch_cuda
    rng = np.random.default_rng(9)
    X = blobs(rng, 2000, 6, 5)
    C = np.vstack([X[:5], np.full((1, 6), 1e3, np.float32)]).astype(np.float64)
    lab, newC, cnt, _ = gpu_kmeans(torch, torch.from_numpy(X).cuda(), C)
    assert cnt[0][5] == 0 and (lab[0] != 5).all() and np.array_equal(newC[5], C[5].astype(np.float32))
    X0 = torch.zeros(0, 6, dtype=torch.float32, device="cuda")
    lab, newC, cnt, inert = gpu_kmeans(torch, X0, C)
    assert lab.size == 0 and (cnt == 0).all() and inert[0] == 0.0
    assert np.array_equal(newC, C.astype(np.float32))


def test_kmeans_deterministic_and_monotone(torch_cuda):
    """Two runs from the same centroids give the same bits; Lloyd iterations
    never raise the inertia (measured under the centroids entering each step)."""
    torch = torch_cuda
    import soft_clustering_em_amd as g
    rng = np.random.default_rng(21)
    X = torch.from_numpy(blobs(rng, 50_000, 32, 64)).cuda()
    C0 = X[torch.from_numpy(rng.choice(50_000, 64, replace=False)).cuda()].contiguous()
    a, b = C0.clone(), C0.clone()
    la, _, ia = g.gmm_kmeans_step(X, a)
    lb, _, ib = g.gmm_kmeans_step(X, b)
    assert torch.equal(a, b) and torch.equal(la, lb) and torch.equal(ia, ib)
    hist = []
    for _ in range(8):
        _, _, inert = g.gmm_kmeans_step(X, a)
        hist.append(float(inert[0]))
    print("inertia", [f"{v:.6g}" for v in hist], flush=True)
    assert all(h1 <= h0 * (1 + 1e-9) for h0, h1 in zip(hist, hist[1:]))


def test_kmeans_estimator_follows_the_oracle(torch_cuda):
    """KMeans from given centres runs the oracle's Lloyd steps: after each
    step the centres agree (the oracle is fed the float32 centres the GPU
    keeps), the inertia history matches, and labels_ are the nearest final
    centres."""
    torch = torch_cuda
    from soft_clustering_em_amd.estimator import KMeans
    rng = np.random.default_rng(31)
    X = blobs(rng, 20_000, 16, 24)
    C0 = X[rng.choice(20_000, 24, replace=False)]
    km = KMeans(24, max_iter=6, tol=0.0, init=C0).fit(torch.from_numpy(X).cuda())
    C = C0.astype(np.float64)
    inert = []
    for _ in range(6):
        lab, gap, newC, cnt, i0 = oracle.kmeans_step(X, C)
        assert decided(X.astype(np.float64), C, gap).all()
        inert.append(i0)
        C = newC.astype(np.float32).astype(np.float64)
    np.testing.assert_allclose(km.cluster_centers_.cpu().numpy(), C.astype(np.float32), rtol=1e-6,
                               atol=1e-6 * np.abs(C).max())
    np.testing.assert_allclose(km.inertia_history_, inert, rtol=1e-9)
    lab, gap, _, cnt, i1 = oracle.kmeans_step(X, km.cluster_centers_.cpu().numpy().astype(np.float64))
    ok = decided(X.astype(np.float64), C, gap)
    assert np.array_equal(km.labels_.cpu().numpy()[ok], lab[ok]) and km.n_iter_ == 6
    assert abs(km.inertia_ - i1) <= 1e-9 * i1


def test_gaussian_mixture_kmeans_init(torch_cuda):
    """init_params="kmeans" starts EM from the Lloyd centres of the same seed
    with weights from the cluster sizes, and the fit then ascends."""
    torch = torch_cuda
    from soft_clustering_em_amd.estimator import GaussianMixture, KMeans
    rng = np.random.default_rng(32)
    X = torch.from_numpy(blobs(rng, 8000, 6, 10)).cuda()
    gm = GaussianMixture(10, covariance_type="diag", max_iter=10, tol=0.0, init_params="kmeans", random_state=4)
    w, mu, cv = gm._init(X)
    km = KMeans(10, max_iter=20, random_state=4).fit(X)
    assert torch.equal(mu, km.cluster_centers_)
    np.testing.assert_allclose(w.cpu().numpy(), km.counts_.cpu().numpy() / 8000.0, rtol=1e-6)
    gm.fit(X)
    h = np.asarray(gm.lower_bound_history_)
    assert (np.diff(h) >= -1e-6 * np.abs(h[1:])).all(), h
