"""The IVF configuration at scale: one EM step of the large-K path (bf16
rows, D = 128, K = 4096; the launch configuration the benchmark times: row
chunks of 2^20, slice-parallel passes) against the float64 oracle on the
workload's first 2^21 + 52,848 rows -- two full chunks and a ragged third,
about 500 rows per component -- from the oracle's own trajectory at t = 0, 1
and 9.  The oracle's outputs come from tests/golden/ivf_bf16_steps.npz,
written by tests/golden/make_ivf_golden.py (which runs only oracle/ and the
input generator); the rows and theta_0 are regenerated here and checked
against the digests stored with them.  Bar: 2e-2 (bf16 rows) on means,
variances, weights (components with oracle N_k >= 1) and the mean LL."""
import hashlib
import os

import numpy as np
import pytest

from parity import TOL_LOWP, param_errors, to_np
from soft_clustering_em_amd import synth

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "ivf_bf16_steps.npz")


def digest(*arrays):
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


@pytest.fixture(scope="module")
def setup():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import soft_clustering_em_amd._abi as abi
    abi.lib()
    ref = np.load(GOLDEN)
    n = int(ref["n_rows"])
    wl = synth.ivf_bf16(N=n)
    th0 = (wl.w0[0].astype(np.float32), wl.mu0[0].astype(np.float32), wl.cv0[0].astype(np.float32))
    assert digest(wl.X) == str(ref["x_sha"]), "regenerated IVF rows differ from the ones the references were made on"
    assert digest(*th0) == str(ref["theta0_sha"]), "regenerated theta_0 differs"
    X = torch.from_numpy(wl.X.view(np.int16)).cuda().view(torch.bfloat16)
    return torch, wl, ref, X, th0


def theta_in(ref, th0, t):
    if t == 0:
        return th0
    if f"in{t}_w" in ref.files:
        return ref[f"in{t}_w"], ref[f"in{t}_mu"], ref[f"in{t}_cv"]
    return ref[f"out{t - 1}_w"], ref[f"out{t - 1}_mu"], ref[f"out{t - 1}_cv"]


@pytest.mark.parametrize("t", [0, 1, 9])
def test_ivf_one_step_at_scale(setup, t):
    import soft_clustering_em_amd as g
    torch, wl, ref, X, th0 = setup
    w, mu, cv = (torch.from_numpy(np.ascontiguousarray(a)[None]).cuda() for a in theta_in(ref, th0, t))
    mll = torch.zeros(1, dtype=torch.float64, device="cuda")
    cs = torch.full((1, wl.K), -1, dtype=torch.int32, device="cuda")
    g.gmm_fit_step(X, w, mu, cv, "spherical", reg_covar=wl.eps, mean_loglik=mll, comp_status=cs)
    torch.cuda.synchronize()
    out = (ref[f"out{t}_w"][None].astype(np.float64), ref[f"out{t}_mu"][None].astype(np.float64),
           ref[f"out{t}_cv"][None].astype(np.float64))
    e = param_errors("spherical", 1, wl.K, wl.D, (to_np(w), to_np(mu), to_np(cv)), out, ref[f"out{t}_nk"][None])
    e_ll = abs(float(mll[0]) - float(ref[f"out{t}_mean_ll"])) / abs(float(ref[f"out{t}_mean_ll"]))
    print(f"IVF N={wl.N} K={wl.K} t={t}: mu={e['mu']:.2e} cv={e['cv']:.2e} w={e['w']:.2e} ll={e_ll:.2e} "
          f"live={e['live']} min var={float(ref[f'out{t}_cv'].min()):.2e}", flush=True)
    assert max(e["mu"], e["cv"], e["w"], e_ll) <= TOL_LOWP, (t, e, e_ll)
    assert (cs.cpu().numpy() >= 0).all()
