"""Parity of gmm_fisher_vector (Fisher vectors of sets of rows under one
diagonal GMM) against the float64 oracle (oracle.fisher_vector), whose
gradient blocks are pinned by central differences of the oracle's mean
log-likelihood.  The GPU statistics are the fused E-step's (float32 logits,
float64 sums), so values agree to about 1e-6 of the vector's scale; the
bar, 1e-4 of the largest entry, is the float32 one."""
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


def model(rng, K, D, X):
    w = rng.dirichlet(np.full(K, 2.0)).astype(np.float32)
    mu = X.reshape(-1, D)[rng.choice(X.reshape(-1, D).shape[0], K, replace=False)].astype(np.float32)
    var = rng.uniform(0.5, 2.0, size=(K, D)).astype(np.float32)
    return w, mu, var


def gpu_fv(torch, X, w, mu, var, power, l2):
    import soft_clustering_em_amd as g
    t = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (X, w, mu, var)]
    fv = g.gmm_fisher_vector(*t, power=power, l2=l2)
    torch.cuda.synchronize()
    return fv.cpu().numpy()


def close(label, got, ref):
    err = np.max(np.abs(got - ref)) / np.max(np.abs(ref))
    print(f"{label}: max |diff| / max |fv| = {err:.2e}", flush=True)
    assert err <= 1e-4, label


@pytest.mark.parametrize("power,l2", [(False, False), (True, True), (True, False), (False, True)])
def test_fisher_vectors_match_the_oracle(torch_cuda, power, l2):
    rng = np.random.default_rng(3)
    B, N, D, K = 5, 777, 13, 9
    X = (rng.normal(size=(B, N, D)) * 1.5 + rng.normal(size=(B, 1, D))).astype(np.float32)
    w, mu, var = model(rng, K, D, X)
    got = gpu_fv(torch_cuda, X, w, mu, var, power, l2)
    ref = oracle.fisher_vector(X, w, mu, var, power=power, l2=l2)
    assert got.shape == (B, 2 * K * D)
    close(f"B={B} N={N} D={D} K={K} power={power} l2={l2}", got, ref)
    if l2:
        np.testing.assert_allclose(np.linalg.norm(got, axis=1), 1.0, rtol=1e-5)


def test_fisher_vectors_batched_equal_single_sets(torch_cuda):
    rng = np.random.default_rng(4)
    B, N, D, K = 4, 1000, 16, 12
    X = rng.normal(size=(B, N, D)).astype(np.float32)
    w, mu, var = model(rng, K, D, X)
    both = gpu_fv(torch_cuda, X, w, mu, var, True, True)
    for b in range(B):
        one = gpu_fv(torch_cuda, X[b], w, mu, var, True, True)
        assert np.array_equal(one[0], both[b]), b


def test_fisher_vectors_sampled_sets_of_a_large_batch(torch_cuda):
    """64 sets of 4096 rows, D = 64, K = 64: three sampled sets against the oracle."""
    rng = np.random.default_rng(5)
    B, N, D, K = 64, 4096, 64, 64
    X = (rng.normal(size=(B, N, D)) + 2.0 * rng.normal(size=(B, 1, D))).astype(np.float32)
    w, mu, var = model(rng, K, D, X)
    got = gpu_fv(torch_cuda, X, w, mu, var, True, True)
    for b in (0, 31, 63):
        ref = oracle.fisher_vector(X[b], w, mu, var)[0]
        close(f"large batch set {b}", got[b], ref)


def test_fisher_vectors_dead_component_and_empty_sets(torch_cuda):
    """A component of weight 0 gives zero blocks; sets of no rows give zeros."""
    torch = torch_cuda
    rng = np.random.default_rng(6)
    B, N, D, K = 2, 500, 5, 4
    X = rng.normal(size=(B, N, D)).astype(np.float32)
    w, mu, var = model(rng, K, D, X)
    w[2] = 0.0
    w /= w.sum()
    got = gpu_fv(torch, X, w, mu, var, False, False)
    KD = K * D
    assert (got[:, 2 * D:3 * D] == 0).all() and (got[:, KD + 2 * D:KD + 3 * D] == 0).all()
    import soft_clustering_em_amd as g
    t = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (w, mu, var)]
    fv = g.gmm_fisher_vector(torch.zeros(3, 0, D, device="cuda"), *t)
    torch.cuda.synchronize()
    assert fv.shape == (3, 2 * KD) and (fv == 0).all()
