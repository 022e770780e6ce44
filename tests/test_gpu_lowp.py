"""16-bit rows beyond the large-K path: IEEE half rows for every covariance
type, and bf16 rows for diagonal, tied and full components and for several
spherical problems, through the fused E-step (rows decoded exactly to float32
as a tile is staged).  One EM step from identical float32 parameters against
the float64 oracle reading the same 16-bit values (its exact decoding is
pinned against numpy for every bit pattern); the bar for 16-bit rows is 2e-2
(the arithmetic after decoding is the float32 path's, so the errors are the
float32 path's too).  Top-m indices bit-exact where the oracle's margin
exceeds 1e-6."""
import numpy as np
import pytest

import oracle
from parity import TOL_LOWP, param_errors, to_np
from soft_clustering_em_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import soft_clustering_em_amd._abi as abi
    abi.lib()
    return torch


def rows16(torch, Xf, kind):
    """(device tensor, oracle input per problem, float64 values)"""
    if kind == "f16":
        h = Xf.astype(np.float16)
        return torch.from_numpy(h).cuda(), [(h[b].view(np.uint16), "f16") for b in range(h.shape[0])], \
            h.astype(np.float64)
    bits = synth.f32_to_bf16_bits(Xf)
    t = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    return t, [(bits[b], "bf16") for b in range(bits.shape[0])], synth.bf16_bits_to_f32(bits).astype(np.float64)


def theta(rng, cov, B, K, D, X64):
    w = np.full((B, K), 1.0 / K, np.float32)
    mu = np.stack([X64[b][rng.choice(X64.shape[1], K, replace=False)] for b in range(B)]).astype(np.float32)
    if cov == "spherical":
        cv = np.ones((B, K), np.float32)
    elif cov == "diag":
        cv = rng.uniform(0.5, 2.0, (B, K, D)).astype(np.float32)
    elif cov == "full":
        cv = np.broadcast_to(np.eye(D, dtype=np.float32), (B, K, D, D)).copy()
    else:
        cv = np.broadcast_to(np.eye(D, dtype=np.float32), (B, D, D)).copy()
    return w, mu, cv


def step_and_check(torch, label, X, Xo, cov, th, B, K, D):
    import soft_clustering_em_amd as g
    w, mu, cv = (torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in th)
    mll = torch.zeros(B, dtype=torch.float64, device="cuda")
    g.gmm_fit_step(X, w, mu, cv, cov, mean_loglik=mll)
    torch.cuda.synchronize()
    got = (to_np(w), to_np(mu), to_np(cv))
    for b in range(B):
        o = oracle.fit_step(cov, Xo[b], *(a[b].astype(np.float64) for a in th))
        e = param_errors(cov, 1, K, D, tuple(a[b] for a in got), (o["w"], o["mu"], o["cv"]), o["stats"]["nk"])
        e_ll = abs(float(mll[b]) - o["mean_ll"][0]) / abs(o["mean_ll"][0])
        print(f"{label} b={b}: mu={e['mu']:.1e} cv={e['cv']:.1e} w={e['w']:.1e} ll={e_ll:.1e}", flush=True)
        assert max(e["mu"], e["cv"], e["w"], e_ll) <= TOL_LOWP, (label, b, e, e_ll)


@pytest.mark.parametrize("kind,cov,B,N,D,K", [
    ("f16", "spherical", 1, 20_000, 32, 48), ("f16", "diag", 2, 15_003, 64, 64), ("f16", "full", 1, 12_000, 16, 12),
    ("f16", "tied", 2, 8_000, 8, 10), ("f16", "spherical", 3, 4_001, 128, 256),
    ("bf16", "diag", 1, 20_000, 64, 256), ("bf16", "diag", 3, 5_000, 20, 30), ("bf16", "full", 2, 10_000, 12, 9),
    ("bf16", "tied", 1, 9_000, 16, 7), ("bf16", "spherical", 2, 6_000, 40, 50)])
def test_16bit_rows_one_step(torch_cuda, kind, cov, B, N, D, K):
    rng = np.random.default_rng(N + D + K)
    centers = 3.0 * rng.standard_normal((B, K, D))
    lab = rng.integers(0, K, (B, N))
    Xf = (np.take_along_axis(centers, lab[..., None], 1) + rng.uniform(0.5, 1.5) * rng.standard_normal((B, N, D)))
    X, Xo, X64 = rows16(torch_cuda, Xf.astype(np.float32), kind)
    step_and_check(torch_cuda, f"{kind} {cov} B={B} N={N} D={D} K={K}", X, Xo, cov, theta(rng, cov, B, K, D, X64),
                   B, K, D)


def test_half_rows_of_the_diagonal_workload(torch_cuda):
    """The diagonal workload (means ~ N(0, 4I), per-dimension std 0.3-1.5,
    Dirichlet weights, k-means++ start) at 200,000 rows, stored as half."""
    wl = synth.diag_large(N=200_000)
    X, Xo, _ = rows16(torch_cuda, wl.X, "f16")
    step_and_check(torch_cuda, "f16 diag_large N=200k", X, Xo, "diag", (wl.w0, wl.mu0, wl.cv0), 1, wl.K, wl.D)


@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_16bit_rows_top_m(torch_cuda, kind):
    """Diagonal components over 16-bit rows (bf16 diag takes the fused top-m
    kernel): ranks exact where the oracle's margin exceeds 1e-6."""
    import soft_clustering_em_amd as g
    torch = torch_cuda
    rng = np.random.default_rng(17)
    N, D, K, m, thr = 8000, 24, 40, 4, 0.05
    centers = 2.0 * rng.standard_normal((K, D))
    Xf = (centers[rng.integers(0, K, N)] + rng.standard_normal((N, D))).astype(np.float32)[None]
    X, Xo, X64 = rows16(torch, Xf, kind)
    w, mu, cv = theta(rng, "diag", 1, K, D, X64)
    idx = torch.empty((1, N, m), dtype=torch.int32, device="cuda")
    resp = torch.empty((1, N, m), dtype=torch.float32, device="cuda")
    cnt = torch.empty((1, N), dtype=torch.int32, device="cuda")
    g.gmm_predict_proba_topm(X, *(torch.from_numpy(a).cuda() for a in (w, mu, cv)), "diag", m, thr, idx, resp, cnt)
    torch.cuda.synchronize()
    oi, orr, oc, _, om = oracle.topm("diag", Xo[0], w[0].astype(np.float64), mu[0].astype(np.float64),
                                     cv[0].astype(np.float64), m, float(np.float32(thr)))
    ok = om > 1e-6
    gi, gc = idx.cpu().numpy()[0], cnt.cpu().numpy()[0]
    assert (~ok).sum() <= max(2, 0.001 * N)
    assert ((gi != oi).any(1) & ok).sum() == 0
    assert ((gc != oc) & ok).sum() == 0
    kept = (oi >= 0) & ok[:, None]
    np.testing.assert_allclose(resp.cpu().numpy()[0][kept], orr[kept], rtol=1e-6, atol=1e-7)


def test_half_rows_top_k_and_streamed(torch_cuda):
    """The top-k EM step and the streamed fit step over half rows."""
    import soft_clustering_em_amd as g
    torch = torch_cuda
    rng = np.random.default_rng(23)
    N, D, K = 12_000, 16, 32
    centers = 3.0 * rng.standard_normal((K, D))
    Xf = (centers[rng.integers(0, K, N)] + rng.standard_normal((N, D))).astype(np.float32)[None]
    X, Xo, X64 = rows16(torch, Xf, "f16")
    th = theta(rng, "diag", 1, K, D, X64)
    # top-k, k = 3
    w, mu, cv = (torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in th)
    g.gmm_topk_fit_step(X, w, mu, cv, "diag", 3)
    torch.cuda.synchronize()
    ref = oracle.topk_fit_step("diag", Xo[0], *(a[0].astype(np.float64) for a in th), 3)
    e = param_errors("diag", 1, K, D, (to_np(w), to_np(mu), to_np(cv)), (ref["w"], ref["mu"], ref["cv"]),
                     ref["stats"]["nk"])
    print(f"f16 top-k: {e}", flush=True)
    assert max(e["mu"], e["cv"], e["w"]) <= TOL_LOWP
    # streamed from pinned host memory, chunks of 5000 rows
    Xh = torch.empty(X.shape, dtype=torch.float16, pin_memory=True)
    Xh.copy_(X.cpu())
    w, mu, cv = (torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in th)
    g.gmm_fit_step_streamed(Xh, w, mu, cv, "diag", 5000)
    torch.cuda.synchronize()
    o = oracle.fit_step("diag", Xo[0], *(a[0].astype(np.float64) for a in th))
    e = param_errors("diag", 1, K, D, (to_np(w), to_np(mu), to_np(cv)), (o["w"], o["mu"], o["cv"]), o["stats"]["nk"])
    print(f"f16 streamed: {e}", flush=True)
    assert max(e["mu"], e["cv"], e["w"]) <= TOL_LOWP
