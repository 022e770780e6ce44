"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every symbol include/gmm.h declares, sizes its workspace independently of N,
and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

from soft_clustering_em_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gmm.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gmm_[a-z_]+)\s*\(", src)))


def test_header_declares_the_binding_surface():
    assert declared_functions() == sorted(_abi.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = _abi.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert L.gmm_version() >= 200


def test_struct_layouts_match_the_header():
    # pointer, int32 (+pad), five int64
    assert ctypes.sizeof(_abi.GmmData) == 8 + 8 + 5 * 8
    assert ctypes.sizeof(_abi.GmmParams) == 4 + 4 + 3 * 8
    assert ctypes.sizeof(_abi.GmmStats) == 4 * 8
    assert ctypes.sizeof(_abi.GmmOptions) == 8 + 8 + 2 * 8


def _data(N, D=64, B=1, dtype=_abi.DT_F32, ld=None):
    ld = D if ld is None else ld
    return _abi.GmmData(ctypes.c_void_p(4096), dtype, B, N, D, ld, N * ld)


def test_workspace_does_not_grow_with_n():
    L = _abi.lib()
    sizes = [L.gmm_workspace_bytes(ctypes.byref(_data(n)), 256, _abi.COV_DIAG, _abi.OP_FIT, 0)
             for n in (10 ** 6, 10 ** 7, 10 ** 8, 10 ** 9)]
    assert sizes[0] > 0 and len(set(sizes)) == 1
    # far below the responsibility matrix of the paper's example (N=10M, K=2048, fp32: ~80 GB)
    assert sizes[0] < 10 ** 8


@pytest.mark.parametrize("cov", [0, 1, 2, 3])
def test_workspace_is_aligned_and_positive(cov):
    L = _abi.lib()
    n = L.gmm_workspace_bytes(ctypes.byref(_data(5000, D=16)), 32, cov, _abi.OP_FIT, 0)
    assert n > 0 and n % 256 == 0


def test_unsupported_shapes_report_zero_workspace():
    L = _abi.lib()
    assert L.gmm_workspace_bytes(ctypes.byref(_data(1000, D=129)), 16, _abi.COV_DIAG, _abi.OP_FIT, 0) == 0
    assert L.gmm_workspace_bytes(ctypes.byref(_data(1000, D=17)), 16, _abi.COV_FULL, _abi.OP_FIT, 0) == 0
    assert L.gmm_workspace_bytes(None, 16, _abi.COV_DIAG, _abi.OP_FIT, 0) == 0


def _params(K=4, cov=_abi.COV_DIAG, ptr=4096):
    p = ctypes.c_void_p(ptr)
    return _abi.GmmParams(K, cov, p, p, p)


@pytest.mark.parametrize("case,expect", [
    ("null data", _abi.GMM_ERR_INVALID_ARG),
    ("null params", _abi.GMM_ERR_INVALID_ARG),
    ("K=0", _abi.GMM_ERR_INVALID_ARG),
    ("bad cov", _abi.GMM_ERR_INVALID_ARG),
    ("D=0", _abi.GMM_ERR_INVALID_ARG),
    ("ld_x<D", _abi.GMM_ERR_INVALID_ARG),
    ("null weights", _abi.GMM_ERR_INVALID_ARG),
    ("null ws", _abi.GMM_ERR_WORKSPACE),
    ("misaligned ws", _abi.GMM_ERR_WORKSPACE),
    ("small ws", _abi.GMM_ERR_WORKSPACE),
    ("D=129", _abi.GMM_ERR_UNSUPPORTED),
    ("bad flags", _abi.GMM_ERR_INVALID_ARG),
    ("N=0 fit", _abi.GMM_ERR_INVALID_ARG),
])
def test_fit_step_validation_happens_before_any_device_work(case, expect):
    L = _abi.lib()
    d = _data(1000, D=8)
    p = _params()
    ws, wsn = ctypes.c_void_p(1 << 20), 1 << 40
    opts = _abi.GmmOptions(1e-6, 0, None, None)
    dp, pp = ctypes.byref(d), ctypes.byref(p)
    if case == "null data":
        dp = None
    elif case == "null params":
        pp = None
    elif case == "K=0":
        p.K = 0
    elif case == "bad cov":
        p.cov = 9
    elif case == "D=0":
        d.D = 0
    elif case == "ld_x<D":
        d.ld_x = 4
    elif case == "null weights":
        p.weights = None
    elif case == "null ws":
        ws = None
    elif case == "misaligned ws":
        ws = ctypes.c_void_p((1 << 20) + 8)
    elif case == "small ws":
        wsn = 1024
    elif case == "D=129":
        d.D = d.ld_x = 129
    elif case == "bad flags":
        opts.flags = 1
    elif case == "N=0 fit":
        d.N = 0
    st = L.gmm_fit_step(dp, pp, ctypes.byref(opts), None, None, ws, wsn, None)
    assert st == expect, (case, st, L.gmm_last_error())
    assert L.gmm_last_error().decode()


def test_status_strings():
    L = _abi.lib()
    for s in range(6):
        assert L.gmm_status_str(s).decode() != "unknown status"
    assert L.gmm_status_str(99).decode() == "unknown status"


def test_check_components_reports_not_positive_definite():
    """The host-side summary of comp_status: flags 2 and 4 are GMM_ERR_NOT_PD
    (first such component reported), flag 1 alone is not."""
    import numpy as np
    L = _abi.lib()
    first = ctypes.c_int64(7)
    ok = np.array([0, 1, 0, 1], np.int32)
    assert L.gmm_check_components(ok.ctypes.data, ok.size, ctypes.byref(first)) == _abi.GMM_OK
    assert first.value == -1
    for flag in (2, 4, 6):
        bad = np.array([1, 0, flag, 4], np.int32)
        st = L.gmm_check_components(bad.ctypes.data, bad.size, ctypes.byref(first))
        assert st == _abi.GMM_ERR_NOT_PD and first.value == 2
        assert "positive definite" in L.gmm_last_error().decode()
    assert L.gmm_check_components(None, 3, None) == _abi.GMM_ERR_INVALID_ARG
    assert L.gmm_check_components(ok.ctypes.data, 0, None) == _abi.GMM_OK


def test_mstep_validation():
    L = _abi.lib()
    p = _params(cov=_abi.COV_FULL)
    st = _abi.GmmStats(ctypes.c_void_p(4096), ctypes.c_void_p(4096), ctypes.c_void_p(4096), None)
    assert L.gmm_mstep(1, 32, ctypes.byref(st), 100, ctypes.byref(p), None, None, None) == _abi.GMM_ERR_UNSUPPORTED
    assert L.gmm_mstep(1, 8, ctypes.byref(st), 0, ctypes.byref(p), None, None, None) == _abi.GMM_ERR_INVALID_ARG
    st.nk = None
    assert L.gmm_mstep(1, 8, ctypes.byref(st), 100, ctypes.byref(p), None, None, None) == _abi.GMM_ERR_INVALID_ARG


# ------------------------------------------------------------------ bf16 rows (large-K path)
def _bf16(N, D=128, B=1):
    return _data(N, D=D, B=B, dtype=_abi.DT_BF16)


@pytest.mark.parametrize("cov,B,D,K,ok,ok16", [
    (_abi.COV_SPHERICAL, 1, 128, 4096, True, True),    # bf16: large-K path; half rows: the fused path in blocks
    (_abi.COV_SPHERICAL, 1, 100, 300, True, True),
    (_abi.COV_SPHERICAL, 1, 128, 16384, True, False),   # half rows: above the blocked window (K <= 8192)
    (_abi.COV_SPHERICAL, 1, 128, 16385, False, False),  # above the large-K window
    (_abi.COV_SPHERICAL, 1, 129, 64, False, False),     # D > 128
    (_abi.COV_SPHERICAL, 2, 64, 64, True, True),        # several problems: the fused path
    (_abi.COV_SPHERICAL, 2, 64, 300, True, True),       # ... in blocks above 256 components
    (_abi.COV_SPHERICAL, 2, 64, 8193, False, False),    # ... up to 8192
    (_abi.COV_DIAG, 1, 64, 64, True, True),
    (_abi.COV_DIAG, 3, 128, 40, True, True),
    (_abi.COV_FULL, 1, 8, 8, True, True),
    (_abi.COV_TIED, 2, 16, 12, True, True),
    (_abi.COV_FULL, 1, 17, 8, False, False),            # full/tied: D <= 16
])
def test_16bit_support_window(cov, B, D, K, ok, ok16):
    """bf16 rows of one problem with spherical components take the large-K
    path (K <= 16384); every other bf16 case and all half rows take the fused
    path (its K and D window: spherical and diagonal components in blocks up to
    K = 8192, full and tied within one workgroup), the rows decoded exactly to
    float32."""
    L = _abi.lib()
    n = L.gmm_workspace_bytes(ctypes.byref(_bf16(10_000, D=D, B=B)), K, cov, _abi.OP_FIT, 0)
    assert (n > 0) == ok
    f16 = _data(10_000, D=D, B=B, dtype=_abi.DT_F16)
    assert (L.gmm_workspace_bytes(ctypes.byref(f16), K, cov, _abi.OP_FIT, 0) > 0) == ok16


def test_bf16_workspace_stops_growing_after_one_chunk():
    """The large-K scratch is O(rows per chunk): constant once N exceeds a chunk
    (2^20 rows for the fit, 2^18 for top-m)."""
    L = _abi.lib()
    for op, chunk in ((_abi.OP_FIT, 1 << 20), (_abi.OP_TOPM, 1 << 18)):
        sizes = [L.gmm_workspace_bytes(ctypes.byref(_bf16(n)), 4096, _abi.COV_SPHERICAL, op, 4)
                 for n in (chunk, 2 * chunk, 10 ** 7, 10 ** 9)]
        assert len(set(sizes)) == 1, (op, sizes)
        small = L.gmm_workspace_bytes(ctypes.byref(_bf16(chunk // 4)), 4096, _abi.COV_SPHERICAL, op, 4)
        assert 0 < small < sizes[0]
        # far below the float32 N x K responsibility matrix of one chunk
        assert sizes[0] < chunk * 4096 * 4


def test_bf16_small_workspace_is_accepted_down_to_one_tile():
    """A workspace below the preferred size streams shorter chunks; below the
    size for a single 32-row tile the call is rejected before any device work."""
    L = _abi.lib()
    d = _bf16(100_000)
    p = _params(K=4096, cov=_abi.COV_SPHERICAL)
    full = L.gmm_workspace_bytes(ctypes.byref(d), 4096, _abi.COV_SPHERICAL, _abi.OP_FIT, 0)
    tiny = L.gmm_workspace_bytes(ctypes.byref(_bf16(32)), 4096, _abi.COV_SPHERICAL, _abi.OP_FIT, 0)
    opts = _abi.GmmOptions(1e-6, 0, None, None)
    ws = ctypes.c_void_p(1 << 20)
    st = L.gmm_fit_step(ctypes.byref(d), ctypes.byref(p), ctypes.byref(opts), None, None, ws, tiny - 256, None)
    assert st == _abi.GMM_ERR_WORKSPACE, L.gmm_last_error()
    assert tiny < full


# ---------------------------------------------------------------- IVF lists
def test_ivf_workspace_sizes():
    L = _abi.lib()
    n = L.gmm_ivf_workspace_bytes(1, 10_000_000, 4, 4096)
    # one int32 per (4096-row block, component), rounded up to 256 bytes
    nblk = (10_000_000 + 4095) // 4096
    assert n == -(-nblk * 4096 * 4 // 256) * 256
    assert L.gmm_ivf_workspace_bytes(3, 0, 4, 17) == 256  # N = 0: the minimum
    for bad in [(0, 10, 4, 8), (1, 10, 0, 8), (1, 10, 17, 8), (1, 10, 4, 0), (1, 10, 4, 16385),
                (1, 2 ** 29, 16, 8), (1, -1, 4, 8)]:
        assert L.gmm_ivf_workspace_bytes(*bad) == 0, bad


def test_ivf_lists_rejects_bad_arguments_before_the_device():
    L = _abi.lib()
    p = ctypes.c_void_p(4096)
    ws = ctypes.c_void_p(1 << 20)
    ok = L.gmm_ivf_workspace_bytes(1, 100, 4, 8)
    cases = {
        "m": ((1, 100, 0, 8, p, None, p, p, None, ws, ok, None), _abi.GMM_ERR_INVALID_ARG),
        "K": ((1, 100, 4, 20000, p, None, p, p, None, ws, ok, None), _abi.GMM_ERR_UNSUPPORTED),
        "offsets": ((1, 100, 4, 8, p, None, None, p, None, ws, ok, None), _abi.GMM_ERR_INVALID_ARG),
        "idx": ((1, 100, 4, 8, None, None, p, p, None, ws, ok, None), _abi.GMM_ERR_INVALID_ARG),
        "list_resp": ((1, 100, 4, 8, p, None, p, p, p, ws, ok, None), _abi.GMM_ERR_INVALID_ARG),
        "ws align": ((1, 100, 4, 8, p, None, p, p, None, ctypes.c_void_p(4100), ok, None),
                     _abi.GMM_ERR_WORKSPACE),
        "ws size": ((1, 100, 4, 8, p, None, p, p, None, ws, 0, None), _abi.GMM_ERR_WORKSPACE),
    }
    for name, (args, want) in cases.items():
        assert L.gmm_ivf_lists(*args) == want, name
        assert L.gmm_last_error() != b"", name


def test_gaussian_mixture_host_checks():
    """The class rejects an unknown covariance type, a partial init and use
    before fit, on the host."""
    import numpy as np
    import torch
    from soft_clustering_em_amd.estimator import GaussianMixture
    with pytest.raises(ValueError):
        GaussianMixture(4, covariance_type="isotropic")
    gm = GaussianMixture(4, covariance_type="diag", means_init=np.zeros((4, 3), np.float32))
    with pytest.raises(ValueError):
        gm._init(torch.zeros(10, 3))
    with pytest.raises(RuntimeError):
        gm.predict(torch.zeros(10, 3))
    with pytest.raises(ValueError):
        gm.fit(torch.zeros(2, 10, 3))
    with pytest.raises(ValueError):
        GaussianMixture(4, init_params="kmeans++")
    from soft_clustering_em_amd.estimator import KMeans
    with pytest.raises(RuntimeError):
        KMeans(3).predict(torch.zeros(10, 3))
    with pytest.raises(ValueError):
        KMeans(20)._start(torch.zeros(10, 3))


def test_kmeans_workspace_and_window():
    """The k-means step takes the top-m window (float32 and half rows, and bf16
    rows of several problems: K <= 256; bf16 rows of one problem: any K) and a
    workspace that grows with N (posting lists and one responsibility per
    row); sizes are 256-byte multiples."""
    L = _abi.lib()
    for N, D, K in [(10_000, 8, 16), (1_000_000, 64, 256), (5003, 7, 1)]:
        n = L.gmm_kmeans_workspace_bytes(ctypes.byref(_data(N, D)), K)
        assert n > 0 and n % 256 == 0
        assert n >= N * 8
    assert L.gmm_kmeans_workspace_bytes(ctypes.byref(_data(1000, 64)), 257) > 0  # the exact top-m kernel
    assert L.gmm_kmeans_workspace_bytes(ctypes.byref(_data(1000, 64)), 8193) == 0
    assert L.gmm_kmeans_workspace_bytes(ctypes.byref(_data(1000, 64)), 0) == 0
    bf = _data(100_000, 128, dtype=_abi.DT_BF16)
    assert L.gmm_kmeans_workspace_bytes(ctypes.byref(bf), 4096) > 0
    assert L.gmm_kmeans_workspace_bytes(ctypes.byref(_data(1000, 128, B=2, dtype=_abi.DT_BF16)), 64) > 0
    assert L.gmm_kmeans_workspace_bytes(ctypes.byref(_data(1000, 128, B=2, dtype=_abi.DT_BF16)), 300) > 0
    assert L.gmm_kmeans_workspace_bytes(ctypes.byref(_data(1000, 128, B=2, dtype=_abi.DT_BF16)), 8193) == 0
    assert L.gmm_kmeans_workspace_bytes(ctypes.byref(_data(1000, 64, dtype=_abi.DT_F16)), 200) > 0
    a = L.gmm_kmeans_workspace_bytes(ctypes.byref(_data(100_000, 32)), 64)
    b = L.gmm_kmeans_workspace_bytes(ctypes.byref(_data(200_000, 32)), 64)
    assert b > a


def test_kmeans_rejects_bad_arguments_before_the_device():
    L = _abi.lib()
    d = _data(1000, 16)
    n = L.gmm_kmeans_workspace_bytes(ctypes.byref(d), 8)
    p = ctypes.c_void_p(4096)
    ws = ctypes.c_void_p(1 << 20)
    cases = {
        "centroids": ((ctypes.byref(d), 8, None, p, None, None, ws, n, None), _abi.GMM_ERR_INVALID_ARG),
        "labels": ((ctypes.byref(d), 8, p, None, None, None, ws, n, None), _abi.GMM_ERR_INVALID_ARG),
        "K": ((ctypes.byref(d), 0, p, p, None, None, ws, n, None), _abi.GMM_ERR_INVALID_ARG),
        "K window": ((ctypes.byref(d), 8193, p, p, None, None, ws, n, None), _abi.GMM_ERR_UNSUPPORTED),
        "ws align": ((ctypes.byref(d), 8, p, p, None, None, ctypes.c_void_p(4100), n, None), _abi.GMM_ERR_WORKSPACE),
        "ws size": ((ctypes.byref(d), 8, p, p, None, None, ws, n - 256, None), _abi.GMM_ERR_WORKSPACE),
    }
    for name, (args, want) in cases.items():
        assert L.gmm_kmeans_step(*args) == want, name
        assert L.gmm_last_error() != b"", name


def test_fisher_vector_rejects_bad_arguments_before_the_device():
    L = _abi.lib()
    d = _data(1000, 16, B=4)
    n = L.gmm_fisher_vector_workspace_bytes(ctypes.byref(d), 8)
    assert n > 0 and n % 256 == 0
    p = ctypes.c_void_p(4096)
    ws = ctypes.c_void_p(1 << 20)
    good = _abi.GmmParams(8, _abi.COV_DIAG, p, p, p)
    sph = _abi.GmmParams(8, _abi.COV_SPHERICAL, p, p, p)
    nul = _abi.GmmParams(8, _abi.COV_DIAG, None, p, p)
    cases = {
        "spherical model": ((ctypes.byref(d), ctypes.byref(sph), 3, p, ws, n, None), _abi.GMM_ERR_UNSUPPORTED),
        "null means": ((ctypes.byref(d), ctypes.byref(nul), 3, p, ws, n, None), _abi.GMM_ERR_INVALID_ARG),
        "flags": ((ctypes.byref(d), ctypes.byref(good), 4, p, ws, n, None), _abi.GMM_ERR_INVALID_ARG),
        "fv": ((ctypes.byref(d), ctypes.byref(good), 3, None, ws, n, None), _abi.GMM_ERR_INVALID_ARG),
        "ws size": ((ctypes.byref(d), ctypes.byref(good), 3, p, ws, n - 256, None), _abi.GMM_ERR_WORKSPACE),
    }
    for name, (args, want) in cases.items():
        assert L.gmm_fisher_vector(*args) == want, name
        assert L.gmm_last_error() != b"", name


def test_topk_fit_step_window_and_arguments():
    L = _abi.lib()
    d = _data(5000, 16)
    assert L.gmm_topk_fit_workspace_bytes(ctypes.byref(d), 32, _abi.COV_DIAG, 4) > 0
    assert L.gmm_topk_fit_workspace_bytes(ctypes.byref(d), 32, _abi.COV_FULL, 4) == 0
    assert L.gmm_topk_fit_workspace_bytes(ctypes.byref(d), 32, _abi.COV_DIAG, 0) == 0
    assert L.gmm_topk_fit_workspace_bytes(ctypes.byref(d), 32, _abi.COV_DIAG, 17) == 0
    a = L.gmm_topk_fit_workspace_bytes(ctypes.byref(d), 32, _abi.COV_DIAG, 2)
    b = L.gmm_topk_fit_workspace_bytes(ctypes.byref(d), 32, _abi.COV_DIAG, 8)
    assert b > a
    p = ctypes.c_void_p(4096)
    prm = _abi.GmmParams(32, _abi.COV_TIED, p, p, p)
    assert L.gmm_topk_fit_step(ctypes.byref(d), ctypes.byref(prm), 4, None, None, None, ctypes.c_void_p(1 << 20),
                               1 << 30, None) == _abi.GMM_ERR_UNSUPPORTED


def test_kde_workspace_size_and_bad_arguments_before_the_device():
    L = _abi.lib()
    d = _data(1000, 5, B=2)
    # D = 5 -> 16 padded features; M = 65 -> two 64-row tiles: mean (256 B aligned),
    # centred references 128 x 16 floats, norms 128 floats
    n = L.gmm_kde_workspace_bytes(ctypes.byref(d), 65)
    assert n == 256 + 128 * 16 * 4 + 512
    assert L.gmm_kde_workspace_bytes(ctypes.byref(d), 0) == 0
    p = ctypes.c_void_p(4096)
    ws = ctypes.c_void_p(1 << 20)
    wide = _data(100, 129)
    half = _data(100, 8, dtype=_abi.DT_BF16)
    cases = {
        "M = 0": ((ctypes.byref(d), p, 0, 5, 1.0, p, ws, n, None), _abi.GMM_ERR_INVALID_ARG),
        "h = 0": ((ctypes.byref(d), p, 65, 5, 0.0, p, ws, n, None), _abi.GMM_ERR_INVALID_ARG),
        "h < 0": ((ctypes.byref(d), p, 65, 5, -1.0, p, ws, n, None), _abi.GMM_ERR_INVALID_ARG),
        "h nan": ((ctypes.byref(d), p, 65, 5, float("nan"), p, ws, n, None), _abi.GMM_ERR_INVALID_ARG),
        "h inf": ((ctypes.byref(d), p, 65, 5, float("inf"), p, ws, n, None), _abi.GMM_ERR_INVALID_ARG),
        "1/(2h^2) overflows": ((ctypes.byref(d), p, 65, 5, 1e-30, p, ws, n, None), _abi.GMM_ERR_INVALID_ARG),
        "ld_ref < D": ((ctypes.byref(d), p, 65, 4, 1.0, p, ws, n, None), _abi.GMM_ERR_INVALID_ARG),
        "null ref": ((ctypes.byref(d), None, 65, 5, 1.0, p, ws, n, None), _abi.GMM_ERR_INVALID_ARG),
        "null out": ((ctypes.byref(d), p, 65, 5, 1.0, None, ws, n, None), _abi.GMM_ERR_INVALID_ARG),
        "ws size": ((ctypes.byref(d), p, 65, 5, 1.0, p, ws, n - 256, None), _abi.GMM_ERR_WORKSPACE),
        "ws align": ((ctypes.byref(d), p, 65, 5, 1.0, p, ctypes.c_void_p((1 << 20) + 64), n, None),
                     _abi.GMM_ERR_WORKSPACE),
        "D > 128": ((ctypes.byref(wide), p, 65, 129, 1.0, p, ws, 1 << 30, None), _abi.GMM_ERR_UNSUPPORTED),
        "bf16 queries": ((ctypes.byref(half), p, 65, 8, 1.0, p, ws, 1 << 30, None), _abi.GMM_ERR_UNSUPPORTED),
    }
    for name, (args, want) in cases.items():
        assert L.gmm_kde_score(*args) == want, name
        assert L.gmm_last_error() != b"", name
    # no query rows: accepted, nothing launched
    e = _data(0, 5)
    assert L.gmm_kde_score(ctypes.byref(e), p, 65, 5, 1.0, None, ws, n, None) == _abi.GMM_OK


def test_noalloc_rejects_a_problem_above_its_static_scratch():
    """1M rows x D = 64, K = 256 diagonal needs about 69 MB of workspace, more
    than the 64 MiB static array: GMM_ERR_WORKSPACE before any device work
    (the pointers are never touched)."""
    L = _abi.lib()
    d = _abi.GmmData(ctypes.c_void_p(4096), _abi.DT_F32, 1, 1_000_000, 64, 64, 0)
    p = _abi.GmmParams(256, _abi.COV_DIAG, ctypes.c_void_p(4096), ctypes.c_void_p(4096), ctypes.c_void_p(4096))
    assert L.gmm_workspace_bytes(ctypes.byref(d), 256, _abi.COV_DIAG, _abi.OP_FIT, 0) > (64 << 20)
    st = L.gmm_fit_step_noalloc(ctypes.byref(d), ctypes.byref(p), None, None, None, None)
    assert st == _abi.GMM_ERR_WORKSPACE
    assert "static" in L.gmm_last_error().decode()


def test_streamed_workspace_depends_on_the_chunk_not_on_n():
    """gmm_fit_step_streamed keeps two chunk buffers and one chunk's scratch:
    its workspace is the same for 10^5 and 10^9 host rows, and grows with the
    chunk size."""
    L = _abi.lib()

    def ws(N, C, dtype=_abi.DT_F32, K=256, cov=_abi.COV_DIAG):
        d = _abi.GmmData(ctypes.c_void_p(4096), dtype, 1, N, 128 if dtype == _abi.DT_BF16 else 64,
                         128 if dtype == _abi.DT_BF16 else 64, 0)
        return L.gmm_fit_step_streamed_workspace_bytes(ctypes.byref(d), K, cov, C)

    assert ws(10**5, 1 << 16) == ws(10**9, 1 << 16) > 0
    assert ws(10**9, 1 << 17) > ws(10**9, 1 << 16)
    assert ws(10**5, 1 << 16, _abi.DT_BF16, 4096, _abi.COV_SPHERICAL) == ws(10**9, 1 << 16, _abi.DT_BF16, 4096,
                                                                            _abi.COV_SPHERICAL) > 0
    assert ws(10**9, 0) == 0  # chunk_rows must be >= 1
