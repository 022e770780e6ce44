"""Writes tests/golden/ivf_bf16_steps.npz: one-step references of the float64
oracle on the IVF workload (spherical components over bf16 rows, D = 128,
K = 4096), at N = 2^21 + 52,848 rows -- two full 2^20-row chunks of the
large-K path and a ragged third.

The trajectory is the oracle's own: theta_0 from the workload generator,
theta_{t+1} = the float32 rounding of one float64 oracle EM step from theta_t
(Flash-GMM, Section 2: E-step scores, log-sum-exp responsibilities, M-step
eqs. 1-3).  For t in STEPS the file keeps the step's output (w, mu, var as
float32 -- their rounding, 6e-8 relative, is far below the bf16 bar of 2e-2),
the oracle's N_k (float64, which components the mean / variance checks cover)
and the mean log-likelihood of theta_t (float64).  The inputs of t = 0 come
from the generator, those of t = 1 are the output of t = 0, and those of the
last t are stored.  sha256 digests of the rows and of theta_0 let a test
confirm it regenerated the same inputs.

Only oracle/ and the input generator run here; nothing of the HIP library.
Run from the repository root:  python tests/golden/make_ivf_golden.py
(about 10 oracle steps of 2.15M x 4096 pairs: an hour or more on 8 cores).
"""
from __future__ import annotations

import hashlib
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from soft_clustering_em_amd import synth  # noqa: E402

N_ROWS = (1 << 21) + 52_848
STEPS = (0, 1, 9)
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "ivf_bf16_steps.npz")


def digest(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def main(nthreads: int = 0) -> None:
    wl = synth.ivf_bf16(N=N_ROWS)
    X = wl.oracle_x()
    th = (wl.w0[0].astype(np.float32), wl.mu0[0].astype(np.float32), wl.cv0[0].astype(np.float32))
    store = dict(n_rows=np.int64(N_ROWS), steps=np.array(STEPS, np.int64), x_sha=np.array(digest(wl.X)),
                 theta0_sha=np.array(digest(*th)))
    for t in range(max(STEPS) + 1):
        t0 = time.time()
        out = oracle.fit_step("spherical", X, *(a.astype(np.float64) for a in th), eps=wl.eps, nthreads=nthreads)
        nxt = (out["w"][0].astype(np.float32), out["mu"][0].astype(np.float32), out["cv"][0].astype(np.float32))
        if t in STEPS:
            if t == max(STEPS) and t - 1 not in STEPS:
                store.update({f"in{t}_w": th[0], f"in{t}_mu": th[1], f"in{t}_cv": th[2]})
            store.update({f"out{t}_w": nxt[0], f"out{t}_mu": nxt[1], f"out{t}_cv": nxt[2],
                          f"out{t}_nk": out["stats"]["nk"][0], f"out{t}_mean_ll": np.float64(out["mean_ll"][0])})
        print(f"step {t}: mean LL {out['mean_ll'][0]:.9f}, {time.time() - t0:.0f} s", flush=True)
        th = nxt
    np.savez_compressed(OUT, **store)
    print("wrote", OUT)


if __name__ == "__main__":
    main(int(sys.argv[1]) if len(sys.argv) > 1 else 0)
