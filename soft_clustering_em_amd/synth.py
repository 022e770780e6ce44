"""Seeded synthetic workloads and starting parameters.

This module only draws random inputs (Gaussian blobs, initial parameters); it
holds none of the EM arithmetic.  The same bytes feed the HIP library and the
float64 oracle, so neither side depends on how they were drawn.

Workloads (sizes, value distributions and initialisations):
  spherical_small  N=10,000  D=8   K=16   fp32, 10 iterations
  diag_large       N=1,000,000 D=64 K=256 fp32, 20 iterations (k-means++ init)
  ivf_bf16         N=10,000,000 D=128 K=4096 bf16, 10 iterations, top-4 / 0.1
  diag_batched     B=64 x N=65,536 D=32 K=64 fp32, 15 iterations
  full_large       N=2,000,000 D=16 K=32 fp32, 20 iterations
  diag_blocked     the diag_large recipe at K=1024 (components in blocks)
Every size can be overridden (smaller copies are parity cases).

The IVF workload stands in for the approximate-nearest-neighbour training sets
the Flash-GMM paper evaluates on (Section 4); no public dataset is read.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np


@dataclass
class Workload:
    name: str
    cov: str
    X: np.ndarray              # (B,N,D) float32, or uint16 holding bf16 bits
    xdtype: str                # "f32" | "bf16"
    w0: np.ndarray             # (B,K) float32
    mu0: np.ndarray            # (B,K,D) float32
    cv0: np.ndarray            # covariance parameters, float32, shape by type
    iters: int
    eps: float = 1e-6
    topm: Optional[tuple] = None   # (m, threshold)
    meta: dict = field(default_factory=dict)

    @property
    def B(self):
        return self.X.shape[0]

    @property
    def N(self):
        return self.X.shape[1]

    @property
    def D(self):
        return self.X.shape[2]

    @property
    def K(self):
        return self.w0.shape[1]

    def oracle_x(self, b=0, rows=None):
        """The input rows of problem b as the oracle takes them."""
        x = self.X[b] if rows is None else self.X[b][rows]
        return (x, "bf16") if self.xdtype == "bf16" else x


# ------------------------------------------------------------------ encoding
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bfloat16, returned as uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ------------------------------------------------------------------ helpers
def _blobs(rng, centers, stds, labels):
    """centers[l] + stds[l] * z, stds per component (scalar) or per (component, dim)."""
    n, d = labels.shape[0], centers.shape[1]
    z = rng.standard_normal((n, d))
    s = stds[labels]
    if s.ndim == 1:
        s = s[:, None]
    return (centers[labels] + s * z).astype(np.float32)


def kmeanspp_seeds(rng, Xs: np.ndarray, K: int) -> np.ndarray:
    """k-means++ seeding (D^2 sampling, Arthur & Vassilvitskii 2007) on rows Xs."""
    Xs = Xs.astype(np.float64)
    n = Xs.shape[0]
    first = int(rng.integers(n))
    idx = [first]
    d2 = ((Xs - Xs[first]) ** 2).sum(1)
    for _ in range(1, K):
        tot = d2.sum()
        if tot <= 0:
            j = int(rng.integers(n))
        else:
            j = int(rng.choice(n, p=d2 / tot))
        idx.append(j)
        d2 = np.minimum(d2, ((Xs - Xs[j]) ** 2).sum(1))
    return np.array(idx)


# ------------------------------------------------------------------ workloads
def spherical_small(N=10_000, D=8, K=16, seed=0, iters=10) -> Workload:
    """16 centres uniform in [-10,10]^D, isotropic std U[0.5,2], equal weights;
    init: K distinct random data points, variance 1, weights 1/K."""
    rng = np.random.default_rng(seed)
    centers = rng.uniform(-10, 10, (K, D))
    stds = rng.uniform(0.5, 2.0, K)
    labels = rng.integers(0, K, N)
    X = _blobs(rng, centers, stds, labels)
    pick = rng.choice(N, K, replace=False)
    mu0 = X[pick].astype(np.float32)
    return Workload("spherical_small", "spherical", X[None], "f32",
                    np.full((1, K), 1.0 / K, np.float32), mu0[None],
                    np.ones((1, K), np.float32), iters)


def diag_large(N=1_000_000, D=64, K=256, seed=0, iters=20, sub=10_000) -> Workload:
    """Means ~ N(0,4I), per-dim std U[0.3,1.5], Dirichlet(2) weights;
    init: k-means++ on a seeded 10k subsample, variance = subsample per-dim
    variance, weights 1/K."""
    rng = np.random.default_rng(seed)
    centers = 2.0 * rng.standard_normal((K, D))
    stds = rng.uniform(0.3, 1.5, (K, D))
    pis = rng.dirichlet(np.full(K, 2.0))
    labels = rng.choice(K, N, p=pis)
    X = np.empty((N, D), np.float32)
    step = 1 << 18
    for s in range(0, N, step):
        X[s:s + step] = _blobs(rng, centers, stds, labels[s:s + step])
    sidx = rng.choice(N, min(sub, N), replace=False)
    Xs = X[sidx]
    seeds = kmeanspp_seeds(rng, Xs, K)
    mu0 = Xs[seeds].astype(np.float32)
    var = Xs.astype(np.float64).var(0)
    cv0 = np.broadcast_to(var.astype(np.float32), (K, D)).copy()
    return Workload("diag_large", "diag", X[None], "f32", np.full((1, K), 1.0 / K, np.float32),
                    mu0[None], cv0[None], iters)


def diag_blocked(N=1_000_000, D=64, K=1024, seed=0, iters=20, sub=10_000) -> Workload:
    """The diag_large recipe with K = 1024 components: more than one
    workgroup holds, so the E-step runs in blocks of components."""
    wl = diag_large(N=N, D=D, K=K, seed=seed, iters=iters, sub=sub)
    return Workload("diag_blocked", wl.cov, wl.X, wl.xdtype, wl.w0, wl.mu0, wl.cv0, wl.iters)


def diag_batched(B=64, N=65_536, D=32, K=64, seed=0, iters=15) -> Workload:
    """Per problem: means ~ N(0,9I), per-dim std U[0.5,1.5], equal weights;
    init per problem: K random points, variance 1, weights 1/K."""
    rng = np.random.default_rng(seed)
    X = np.empty((B, N, D), np.float32)
    mu0 = np.empty((B, K, D), np.float32)
    for b in range(B):
        centers = 3.0 * rng.standard_normal((K, D))
        stds = rng.uniform(0.5, 1.5, (K, D))
        labels = rng.integers(0, K, N)
        X[b] = _blobs(rng, centers, stds, labels)
        mu0[b] = X[b][rng.choice(N, K, replace=False)]
    return Workload("diag_batched", "diag", X, "f32", np.full((B, K), 1.0 / K, np.float32),
                    mu0, np.ones((B, K, D), np.float32), iters)


def full_large(N=2_000_000, D=16, K=32, seed=0, iters=20) -> Workload:
    """Means ~ N(0,16I), Sigma_k = A A^T + 0.1 I with A_ij ~ N(0, 0.5) (variance
    0.5), Dirichlet(1) weights; init: K random points, Sigma = global sample
    covariance, weights 1/K."""
    rng = np.random.default_rng(seed)
    centers = 4.0 * rng.standard_normal((K, D))
    A = np.sqrt(0.5) * rng.standard_normal((K, D, D))
    Sig = A @ A.transpose(0, 2, 1) + 0.1 * np.eye(D)
    Lc = np.linalg.cholesky(Sig)
    pis = rng.dirichlet(np.ones(K))
    labels = rng.choice(K, N, p=pis)
    X = np.empty((N, D), np.float32)
    step = 1 << 18
    for s in range(0, N, step):
        lab = labels[s:s + step]
        z = rng.standard_normal((lab.shape[0], D))
        X[s:s + step] = (centers[lab] + np.einsum("nij,nj->ni", Lc[lab], z)).astype(np.float32)
    mu0 = X[rng.choice(N, K, replace=False)].astype(np.float32)
    C = np.cov(X.astype(np.float64).T, bias=True)
    cv0 = np.broadcast_to(C.astype(np.float32), (K, D, D)).copy()
    return Workload("full_large", "full", X[None], "f32", np.full((1, K), 1.0 / K, np.float32),
                    mu0[None], cv0[None], iters)


def _ivf_blobs(D, K, seed):
    crng = np.random.default_rng([seed, 0])
    centers = crng.standard_normal((K, D))
    centers /= np.linalg.norm(centers, axis=1, keepdims=True)
    stds = crng.uniform(0.05, 0.2, (K, D))
    return centers.astype(np.float32), stds.astype(np.float32)


def _ivf_chunk(c, chunk, D, K, seed, noise, centers, stds):
    """All rows of chunk c (float32), from the chunk's own seed."""
    rng = np.random.default_rng([seed, 1, c])
    labels = rng.integers(0, K, chunk)
    is_noise = rng.random(chunk) < noise
    z = rng.standard_normal((chunk, D), dtype=np.float32)
    rows = centers[labels]
    rows += stds[labels] * z
    rows[is_noise] = rng.standard_normal((int(is_noise.sum()), D), dtype=np.float32)
    rows /= np.linalg.norm(rows, axis=1, keepdims=True)
    return rows


def _workers():
    return max(1, min(16, os.cpu_count() or 1))


def ivf_rows(n_rows: int, start: int, D=128, K=4096, seed=0, noise=0.10, chunk=1 << 16):
    """Rows [start, start+n_rows) of the IVF workload as float32 (before bf16).

    Rows are drawn in independent chunks of `chunk` rows, each from its own
    seed, so any range can be regenerated without the rows before it.
    Blob centres are uniform on the unit sphere with per-(blob, dim) std
    U[0.05,0.2]; `noise` of the rows are standard normal (uniform direction);
    every row is normalised to unit length.
    """
    centers, stds = _ivf_blobs(D, K, seed)
    out = np.empty((n_rows, D), np.float32)
    c0, c1 = start // chunk, (start + n_rows - 1) // chunk

    def one(c):
        lo = c * chunk
        a, b = max(lo, start), min(lo + chunk, start + n_rows)
        out[a - start:b - start] = _ivf_chunk(c, chunk, D, K, seed, noise, centers, stds)[a - lo:b - lo]

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(one, range(c0, c1 + 1)))
    return out


def ivf_bf16(N=10_000_000, D=128, K=4096, seed=0, iters=10, chunk=1 << 16) -> Workload:
    """Unit-normalised mixture of K anisotropic blobs plus 10% uniform-on-sphere
    noise, stored as bf16 (round-to-nearest-even).  Init: K distinct random
    rows, variance = global mean per-dimension variance, weights 1/K."""
    centers, stds = _ivf_blobs(D, K, seed)
    X = np.empty((N, D), np.uint16)
    nchunks = (N + chunk - 1) // chunk

    def one(c):
        s = c * chunk
        n = min(chunk, N - s)
        bits = f32_to_bf16_bits(_ivf_chunk(c, chunk, D, K, seed, 0.10, centers, stds)[:n])
        X[s:s + n] = bits
        v = bf16_bits_to_f32(bits).astype(np.float64)
        return v.sum(0), (v * v).sum(0)

    with ThreadPoolExecutor(_workers()) as ex:
        parts = list(ex.map(one, range(nchunks)))
    s1 = np.sum([p[0] for p in parts], axis=0)   # chunk order: independent of the thread count
    s2 = np.sum([p[1] for p in parts], axis=0)
    mean = s1 / N
    var = float((s2 / N - mean * mean).mean())
    rng = np.random.default_rng([seed, 2])
    pick = rng.choice(N, K, replace=False)
    mu0 = bf16_bits_to_f32(X[np.sort(pick)])
    return Workload("ivf_bf16", "spherical", X[None], "bf16", np.full((1, K), 1.0 / K, np.float32),
                    mu0[None].astype(np.float32), np.full((1, K), var, np.float32), iters,
                    topm=(4, 0.1), meta=dict(chunk=chunk))


def kde_inputs(N=1_000_000, M=65_536, D=64, seed=0, offset=0.0):
    """Kernel density inputs: N query rows and M reference rows drawn from the
    same blob mixture as diag_large (means ~ N(0, 4I), per-dimension std
    U[0.3, 1.5], Dirichlet(2) weights, K = 256 blobs), shifted by `offset` in
    every dimension; bandwidth by Scott's rule, h = s M^(-1/(D+4)) with s the
    root mean per-dimension variance of the references.  Returns (Y (N, D),
    X (M, D)) float32 and h."""
    rng = np.random.default_rng([seed, 7])
    K = 256
    centers = 2.0 * rng.standard_normal((K, D)) + offset
    stds = rng.uniform(0.3, 1.5, (K, D))
    pis = rng.dirichlet(np.full(K, 2.0))
    X = _blobs(rng, centers, stds, rng.choice(K, M, p=pis))
    Y = np.empty((N, D), np.float32)
    step = 1 << 18
    for s0 in range(0, N, step):
        Y[s0:s0 + step] = _blobs(rng, centers, stds, rng.choice(K, min(step, N - s0), p=pis))
    s = float(np.sqrt(X.astype(np.float64).var(0).mean()))
    return Y, X, s * M ** (-1.0 / (D + 4))


WORKLOADS = {
    "spherical_small": spherical_small,
    "diag_large": diag_large,
    "ivf_bf16": ivf_bf16,
    "diag_batched": diag_batched,
    "full_large": full_large,
    "diag_blocked": diag_blocked,
}
