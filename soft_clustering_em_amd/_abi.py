"""ctypes mirror of include/gmm.h and the loader of libgmm.so.

Argument marshalling only: every computation runs in the HIP library.  The
library must have been built (``python -m soft_clustering_em_amd.build`` or
``__graft_entry__.build()``); there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgmm.so")

# enums (include/gmm.h)
COV_SPHERICAL, COV_DIAG, COV_TIED, COV_FULL = 0, 1, 2, 3
COV_CODES = {"spherical": COV_SPHERICAL, "diag": COV_DIAG, "tied": COV_TIED, "full": COV_FULL}
DT_F32, DT_BF16, DT_F16 = 0, 1, 2
OP_FIT, OP_ESTEP, OP_TOPM = 0, 1, 2
GMM_OK, GMM_ERR_INVALID_ARG, GMM_ERR_UNSUPPORTED, GMM_ERR_WORKSPACE, GMM_ERR_HIP, GMM_ERR_NOT_PD = 0, 1, 2, 3, 4, 5

EXPORTED = ["gmm_workspace_bytes", "gmm_estep_stats", "gmm_mstep", "gmm_fit_step", "gmm_fit", "gmm_fit_step_noalloc",
            "gmm_fit_step_streamed_workspace_bytes", "gmm_fit_step_streamed",
            "gmm_predict_proba_topm", "gmm_ivf_workspace_bytes", "gmm_ivf_lists", "gmm_kmeans_workspace_bytes",
            "gmm_kmeans_step", "gmm_fisher_vector_workspace_bytes", "gmm_fisher_vector",
            "gmm_topk_fit_workspace_bytes", "gmm_topk_fit_step", "gmm_kde_workspace_bytes", "gmm_kde_score",
            "gmm_check_components", "gmm_status_str",
            "gmm_last_error", "gmm_version"]


class GmmData(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("B", ctypes.c_int64),
                ("N", ctypes.c_int64), ("D", ctypes.c_int64), ("ld_x", ctypes.c_int64),
                ("stride_b", ctypes.c_int64)]


class GmmParams(ctypes.Structure):
    _fields_ = [("K", ctypes.c_int32), ("cov", ctypes.c_int32), ("weights", ctypes.c_void_p),
                ("means", ctypes.c_void_p), ("covars", ctypes.c_void_p)]


class GmmStats(ctypes.Structure):
    _fields_ = [("nk", ctypes.c_void_p), ("sx", ctypes.c_void_p), ("sxx", ctypes.c_void_p),
                ("loglik", ctypes.c_void_p)]


class GmmOptions(ctypes.Structure):
    _fields_ = [("reg_covar", ctypes.c_double), ("flags", ctypes.c_uint32),
                ("event_begin", ctypes.c_void_p), ("event_end", ctypes.c_void_p)]


class GmmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"gmm status {status}: {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libgmm.so; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build the HIP library first "
                               "(python -m soft_clustering_em_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        L.gmm_workspace_bytes.argtypes = [ctypes.POINTER(GmmData), ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_int32]
        L.gmm_workspace_bytes.restype = ctypes.c_size_t
        L.gmm_estep_stats.argtypes = [ctypes.POINTER(GmmData), ctypes.POINTER(GmmParams),
                                      ctypes.POINTER(GmmStats), ctypes.c_int32, P, ctypes.c_size_t, P]
        L.gmm_mstep.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.POINTER(GmmStats), ctypes.c_int64,
                                ctypes.POINTER(GmmParams), ctypes.POINTER(GmmOptions), P, P]
        L.gmm_fit_step.argtypes = [ctypes.POINTER(GmmData), ctypes.POINTER(GmmParams),
                                   ctypes.POINTER(GmmOptions), P, P, P, ctypes.c_size_t, P]
        L.gmm_fit.argtypes = [ctypes.POINTER(GmmData), ctypes.POINTER(GmmParams), ctypes.POINTER(GmmOptions),
                              ctypes.c_int32, P, P, P, ctypes.c_size_t, P]
        L.gmm_fit_step_noalloc.argtypes = [ctypes.POINTER(GmmData), ctypes.POINTER(GmmParams),
                                           ctypes.POINTER(GmmOptions), P, P, P]
        L.gmm_fit_step_streamed_workspace_bytes.argtypes = [ctypes.POINTER(GmmData), ctypes.c_int32,
                                                            ctypes.c_int32, ctypes.c_int64]
        L.gmm_fit_step_streamed_workspace_bytes.restype = ctypes.c_size_t
        L.gmm_fit_step_streamed.argtypes = [ctypes.POINTER(GmmData), ctypes.POINTER(GmmParams),
                                            ctypes.POINTER(GmmOptions), ctypes.c_int64, P, P, P, ctypes.c_size_t,
                                            P, P]
        L.gmm_predict_proba_topm.argtypes = [ctypes.POINTER(GmmData), ctypes.POINTER(GmmParams),
                                             ctypes.c_int32, ctypes.c_float, P, P, P, P, P,
                                             ctypes.c_size_t, P]
        L.gmm_ivf_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]
        L.gmm_ivf_workspace_bytes.restype = ctypes.c_size_t
        L.gmm_ivf_lists.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, P, P, P, P, P,
                                    P, ctypes.c_size_t, P]
        L.gmm_kmeans_workspace_bytes.argtypes = [ctypes.POINTER(GmmData), ctypes.c_int32]
        L.gmm_kmeans_workspace_bytes.restype = ctypes.c_size_t
        L.gmm_kmeans_step.argtypes = [ctypes.POINTER(GmmData), ctypes.c_int32, P, P, P, P, P, ctypes.c_size_t, P]
        L.gmm_fisher_vector_workspace_bytes.argtypes = [ctypes.POINTER(GmmData), ctypes.c_int32]
        L.gmm_fisher_vector_workspace_bytes.restype = ctypes.c_size_t
        L.gmm_fisher_vector.argtypes = [ctypes.POINTER(GmmData), ctypes.POINTER(GmmParams), ctypes.c_uint32, P, P,
                                        ctypes.c_size_t, P]
        L.gmm_kde_workspace_bytes.argtypes = [ctypes.POINTER(GmmData), ctypes.c_int64]
        L.gmm_kde_workspace_bytes.restype = ctypes.c_size_t
        L.gmm_kde_score.argtypes = [ctypes.POINTER(GmmData), P, ctypes.c_int64, ctypes.c_int64, ctypes.c_double, P, P,
                                    ctypes.c_size_t, P]
        L.gmm_topk_fit_workspace_bytes.argtypes = [ctypes.POINTER(GmmData), ctypes.c_int32, ctypes.c_int32,
                                                   ctypes.c_int32]
        L.gmm_topk_fit_workspace_bytes.restype = ctypes.c_size_t
        L.gmm_topk_fit_step.argtypes = [ctypes.POINTER(GmmData), ctypes.POINTER(GmmParams), ctypes.c_int32,
                                        ctypes.POINTER(GmmOptions), P, P, P, ctypes.c_size_t, P]
        for f in (L.gmm_estep_stats, L.gmm_mstep, L.gmm_fit_step, L.gmm_fit, L.gmm_fit_step_noalloc, L.gmm_fit_step_streamed,
                  L.gmm_predict_proba_topm,
                  L.gmm_ivf_lists,
                  L.gmm_kmeans_step, L.gmm_fisher_vector, L.gmm_topk_fit_step, L.gmm_kde_score):
            f.restype = ctypes.c_int
        L.gmm_check_components.argtypes = [P, ctypes.c_int64, P]
        L.gmm_check_components.restype = ctypes.c_int
        L.gmm_status_str.argtypes = [ctypes.c_int32]
        L.gmm_status_str.restype = ctypes.c_char_p
        L.gmm_last_error.argtypes = []
        L.gmm_last_error.restype = ctypes.c_char_p
        L.gmm_version.argtypes = []
        L.gmm_version.restype = ctypes.c_int32
        _lib = L
    return _lib


def check(status: int) -> None:
    if status != GMM_OK:
        L = lib()
        raise GmmError(status, f"{L.gmm_status_str(status).decode()}: {L.gmm_last_error().decode()}")
