"""GPU parity of the IVF posting lists (gmm_ivf_lists) against the oracle.

The lists are integer work: rows and offsets must be bit-identical to
oracle.ivf_lists, and the copied responsibilities bit-identical to their
sources.  Cases span several 4096-row blocks and 64-row chunks with a ragged
tail, rows that end early (-1 or a value outside [0, K)), several problems,
m from 1 to 16 and K up to 4096; one case starts from a real top-m
assignment, and one checks the full ivf_bf16 workload (N = 10,000,000, m = 4,
K = 4096) through properties that hold at any size.
"""
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


def random_assignment(rng, B, N, m, K, bad_frac=0.02):
    """Top-m-like rows (1..m distinct components, largest responsibility
    first), -1 padded; a few rows end early with a value outside [0, K)."""
    idx = np.full((B, N, m), -1, np.int32)
    resp = np.zeros((B, N, m), np.float32)
    cnt = rng.integers(1, m + 1, size=(B, N))
    for b in range(B):
        for i in range(N):
            c = cnt[b, i]
            idx[b, i, :c] = rng.choice(K, size=c, replace=False) if c <= K else rng.integers(0, K, size=c)
            resp[b, i, :c] = np.sort(rng.random(c).astype(np.float32))[::-1]
    bad = rng.random((B, N)) < bad_frac
    for b, i in zip(*np.nonzero(bad)):
        j = rng.integers(0, m)
        idx[b, i, j] = rng.choice([K, K + 7, -5, 2 ** 30])
    return idx, resp


def gpu_lists(torch, idx, resp, K, with_resp=True):
    import soft_clustering_em_amd as g
    ti = torch.from_numpy(idx).cuda()
    tr = torch.from_numpy(resp).cuda() if with_resp else None
    off, rows, lr = g.gmm_ivf_lists(ti, K, resp=tr)
    torch.cuda.synchronize()
    return off.cpu().numpy(), rows.cpu().numpy(), (lr.cpu().numpy() if lr is not None else None)


def check_against_oracle(torch, idx, resp, K, label):
    off, rows, lr = gpu_lists(torch, idx, resp, K)
    o_off, o_rows, o_lr = oracle.ivf_lists(idx, resp, K)
    B = idx.shape[0]
    print(f"{label}: entries {[int(o_off[b, K]) for b in range(B)]}", flush=True)
    assert np.array_equal(off, o_off), label
    for b in range(B):
        n = int(o_off[b, K])
        assert np.array_equal(rows[b, :n], o_rows[b, :n]), label
        assert np.array_equal(lr[b, :n].view(np.uint32), o_lr[b, :n].view(np.uint32)), label


@pytest.mark.parametrize("B,N,m,K", [(1, 10007, 4, 300), (3, 4097, 3, 7), (1, 9000, 1, 4096),
                                     (2, 4100, 16, 40), (1, 63, 4, 1), (1, 8192, 4, 4096)])
def test_lists_match_oracle(torch_cuda, B, N, m, K):
    rng = np.random.default_rng(N + 31 * m + K)
    idx, resp = random_assignment(rng, B, N, m, K)
    check_against_oracle(torch_cuda, idx, resp, K, f"B={B} N={N} m={m} K={K}")


def test_lists_without_responsibilities(torch_cuda):
    rng = np.random.default_rng(5)
    idx, resp = random_assignment(rng, 1, 5000, 4, 100)
    off, rows, lr = gpu_lists(torch_cuda, idx, resp, 100, with_resp=False)
    o_off, o_rows, _ = oracle.ivf_lists(idx, None, 100)
    assert lr is None
    assert np.array_equal(off, o_off)
    assert np.array_equal(rows[0, :o_off[0, 100]], o_rows[0, :o_off[0, 100]])


def test_empty_input_gives_empty_lists(torch_cuda):
    import soft_clustering_em_amd as g
    torch = torch_cuda
    idx = torch.zeros(2, 0, 4, dtype=torch.int32, device="cuda")
    off, rows, lr = g.gmm_ivf_lists(idx, 9)
    torch.cuda.synchronize()
    assert (off.cpu().numpy() == 0).all()


def test_deterministic_bitwise(torch_cuda):
    rng = np.random.default_rng(11)
    idx, resp = random_assignment(rng, 1, 20000, 4, 512)
    a = gpu_lists(torch_cuda, idx, resp, 512)
    b = gpu_lists(torch_cuda, idx, resp, 512)
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


def test_lists_of_a_real_multi_assignment(torch_cuda):
    """gmm_predict_proba_topm, then the lists of its output, against the
    oracle lists of that same output."""
    import soft_clustering_em_amd as g
    from soft_clustering_em_amd import synth
    torch = torch_cuda
    wl = synth.spherical_small()
    X = torch.from_numpy(wl.X).cuda()
    w, mu, cv = (torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (wl.w0, wl.mu0, wl.cv0))
    m, K = 4, wl.K
    idx = torch.empty(1, wl.N, m, dtype=torch.int32, device="cuda")
    resp = torch.empty(1, wl.N, m, dtype=torch.float32, device="cuda")
    g.gmm_predict_proba_topm(X, w, mu, cv, wl.cov, m, 0.1, idx, resp)
    torch.cuda.synchronize()
    check_against_oracle(torch, idx.cpu().numpy(), resp.cpu().numpy(), K, "spherical_small top-4")


def test_full_size_ivf_lists_properties(torch_cuda):
    """The full ivf_bf16 workload (N = 10,000,000, K = 4096) at its initial
    parameters, top-4 at threshold 0.1, then its lists, in the launch
    configuration the bench times.  Checked through properties that hold at
    any size: offsets are the per-component counts, every list is strictly
    increasing in row, and the (component, row) pairs are exactly those of
    idx; the responsibilities travel with their rows."""
    import soft_clustering_em_amd as g
    from soft_clustering_em_amd import synth
    torch = torch_cuda
    wl = synth.ivf_bf16()
    X = torch.from_numpy(wl.X.view(np.int16)).cuda().view(torch.bfloat16)
    w, mu, cv = (torch.from_numpy(a.copy()).cuda() for a in (wl.w0, wl.mu0, wl.cv0))
    N, K, m = wl.N, wl.K, 4
    idx = torch.empty(1, N, m, dtype=torch.int32, device="cuda")
    resp = torch.empty(1, N, m, dtype=torch.float32, device="cuda")
    g.gmm_predict_proba_topm(X, w, mu, cv, "spherical", m, 0.1, idx, resp)
    del X
    off, rows, lr = g.gmm_ivf_lists(idx, K, resp=resp)
    torch.cuda.synchronize()
    idx, resp = idx.cpu().numpy()[0], resp.cpu().numpy()[0]
    off, rows, lr = off.cpu().numpy()[0], rows.cpu().numpy()[0], lr.cpu().numpy()[0]
    valid = idx >= 0  # top-m output: -1 padding only
    keys = idx[valid]
    n = keys.size
    print(f"full size: {n} entries, {n / N:.3f} per row", flush=True)
    assert off[K] == n
    assert np.array_equal(np.diff(off), np.bincount(keys, minlength=K))
    lk = np.repeat(np.arange(K, dtype=np.int64), np.diff(off))
    r = rows[:n].astype(np.int64)
    # strictly increasing rows inside each list
    inside = lk[1:] == lk[:-1]
    assert (r[1:][inside] > r[:-1][inside]).all()
    # the same (component, row) pairs, ordered by component then row
    rid = np.broadcast_to(np.arange(N, dtype=np.int64)[:, None], idx.shape)[valid]
    order = np.lexsort((rid, keys))
    assert np.array_equal(lk, keys[order].astype(np.int64))
    assert np.array_equal(r, rid[order])
    assert np.array_equal(lr[:n].view(np.uint32), resp[valid][order].view(np.uint32))
