"""CPU oracle of the Polestar-Cache drift-detection path -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It wraps the plain C oracle (``polestar_oracle.c``) with
ctypes; arrays are numpy, host memory, C-contiguous.  bf16 tensors travel as
``numpy.uint16`` bit patterns.

Each function returns the arrays it writes.  Errors raise ``OracleError``.
"""
import ctypes
import os
from dataclasses import dataclass

import numpy as np

from . import build as _build

F32, BF16 = 0, 1
INIT_GIVEN, INIT_STRIDED, INIT_FARTHEST = 0, 1, 2
SCORE_KL_SHARE, SCORE_KL_SHARE_ABS, SCORE_ATTN_WEIGHTED = 0, 1, 2


class OracleError(RuntimeError):
    pass


@dataclass
class Shape:
    W: int
    N: int
    d: int
    Hq: int = 1
    Hkv: int = 1
    dh: int = 16
    Nb: int = 1
    K: int = 1


class _CShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("W", "N", "d", "Hq", "Hkv", "dh", "Nb", "K")]


def _cshape(s: Shape) -> _CShape:
    return _CShape(s.W, s.N, s.d, s.Hq, s.Hkv, s.dh, s.Nb, s.K)


_lib = None


def lib():
    """The oracle's shared library; PSO_ORACLE_LIB names another build of the
    same source to load instead (the sanitizer test's instrumented build)."""
    global _lib
    if _lib is None:
        path = os.environ.get("PSO_ORACLE_LIB") or _build.LIB
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I = ctypes.c_int
        SP = ctypes.POINTER(_CShape)
        L.pso_bf16_to_f32.argtypes, L.pso_bf16_to_f32.restype = [ctypes.c_uint16], ctypes.c_float
        L.pso_f32_to_bf16.argtypes, L.pso_f32_to_bf16.restype = [ctypes.c_float], ctypes.c_uint16
        L.pso_e4m3_decode.argtypes, L.pso_e4m3_decode.restype = [ctypes.c_uint8], ctypes.c_float
        L.pso_e4m3_encode.argtypes, L.pso_e4m3_encode.restype = [ctypes.c_float], ctypes.c_uint8
        L.pso_e2m1_decode.argtypes, L.pso_e2m1_decode.restype = [ctypes.c_uint8], ctypes.c_float
        L.pso_e2m1_encode.argtypes, L.pso_e2m1_encode.restype = [ctypes.c_float], ctypes.c_uint8
        L.pso_row_norms.argtypes = [SP, I, P, P]
        L.pso_kmeans_init.argtypes = [SP, I, P, I, P]
        L.pso_kmeans_fit.argtypes = [SP, I, P, P, I, I, P, P, P, P, P, P]
        L.pso_kmeans_update.argtypes = [SP, I, P, P, P, P, P, P]
        L.pso_residual_nvfp4.argtypes = [SP, I, P, P, P, P, P, P, P]
        L.pso_proxy_attn.argtypes = [SP, I, P, P, ctypes.c_float, P, P, I, P, P, P]
        L.pso_drift_kl.argtypes = [SP, P, P, I, P, P, P]
        L.pso_topk_clusters.argtypes = [SP, P, ctypes.c_int32, P, P]
        L.pso_refresh_gather.argtypes = [SP, I, P, P, ctypes.c_int32, ctypes.c_int32, P, P,
                                         P, P, P, P, P, P, P, P, P, P]
        F = ctypes.c_float
        L.pso_drift_cosine.argtypes = [SP, P, P, P]
        L.pso_commit_block.argtypes = [SP, P, P, ctypes.c_int32, F, F, P, P, P, P]
        L.pso_commit_suffix.argtypes = [SP, P, P, ctypes.c_int32, ctypes.c_int32, P, F, P, P]
        for name in ("pso_drift_cosine", "pso_commit_block", "pso_commit_suffix", "pso_row_norms", "pso_kmeans_init", "pso_kmeans_fit", "pso_kmeans_update",
                     "pso_residual_nvfp4",
                     "pso_proxy_attn", "pso_drift_kl", "pso_topk_clusters", "pso_refresh_gather"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _ok(rc, name):
    if rc != 0:
        raise OracleError(f"{name} returned {rc}")


def _elem(dtype):
    return np.uint16 if dtype == BF16 else np.float32


# ---- number formats ------------------------------------------------------
def bf16_to_f32(b):
    return np.asarray(b, dtype=np.uint16).astype(np.uint32).__lshift__(16).view(np.float32)


def f32_to_bf16(x):
    L = lib()
    x = np.ascontiguousarray(x, dtype=np.float32)
    return np.array([L.pso_f32_to_bf16(float(v)) for v in x.ravel()], dtype=np.uint16).reshape(x.shape)


def e4m3_decode(code):
    return lib().pso_e4m3_decode(int(code))


def e4m3_encode(x):
    return lib().pso_e4m3_encode(float(np.float32(x)))


def e2m1_decode(nib):
    return lib().pso_e2m1_decode(int(nib))


def e2m1_encode(v):
    return lib().pso_e2m1_encode(float(np.float32(v)))


# ---- the path --------------------------------------------------------------
def row_norms(s: Shape, dtype, H):
    out = np.zeros((s.W, s.N), np.float32)
    _ok(lib().pso_row_norms(ctypes.byref(_cshape(s)), dtype, _p(H), _p(out)), "pso_row_norms")
    return out


def kmeans_init(s: Shape, dtype, H, init):
    C = np.zeros((s.W, s.K, s.d), np.float32)
    _ok(lib().pso_kmeans_init(ctypes.byref(_cshape(s)), dtype, _p(H), init, _p(C)), "pso_kmeans_init")
    return C


def kmeans_fit(s: Shape, dtype, H, Kr, init, iters, C, Ck=None):
    """C (and Ck) are updated in place and returned with assign, counts,
    row_norm and objective."""
    assign = np.zeros((s.W, s.N), np.int32)
    counts = np.zeros((s.W, s.K), np.int32)
    rn = np.zeros((s.W, s.N), np.float32)
    obj = np.zeros((s.W,), np.float64)
    if Kr is not None and Ck is None:
        Ck = np.zeros((s.W, s.K, s.Hkv, s.dh), _elem(dtype))
    _ok(lib().pso_kmeans_fit(ctypes.byref(_cshape(s)), dtype, _p(H), _p(Kr), init, iters, _p(C),
                             _p(assign), _p(counts), _p(rn), _p(Ck), _p(obj)), "pso_kmeans_fit")
    return dict(C=C, assign=assign, counts=counts, row_norm=rn, Ck=Ck, objective=obj)


def kmeans_update(s: Shape, dtype, H, row_norm, assign, C):
    """The update step alone from a given assignment; C (in/out) supplies the
    centres that empty clusters keep."""
    C = np.array(C, np.float32, copy=True)
    counts = np.zeros((s.W, s.K), np.int32)
    obj = np.zeros((s.W,), np.float64)
    _ok(lib().pso_kmeans_update(ctypes.byref(_cshape(s)), dtype, _p(H), _p(row_norm), _p(assign),
                                _p(C), _p(counts), _p(obj)), "pso_kmeans_update")
    return dict(C=C, counts=counts, objective=obj)


def residual_nvfp4(s: Shape, dtype, H, row_norm, C, assign):
    codes = np.zeros((s.W, s.N, s.d // 2), np.uint8)
    bscale = np.zeros((s.W, s.N, s.d // 16), np.uint8)
    rscale = np.zeros((s.W, s.N), np.float32)
    _ok(lib().pso_residual_nvfp4(ctypes.byref(_cshape(s)), dtype, _p(H), _p(row_norm), _p(C),
                                 _p(assign), _p(codes), _p(bscale), _p(rscale)), "pso_residual_nvfp4")
    return dict(codes=codes, bscale=bscale, rscale=rscale)


def proxy_attn(s: Shape, dtype, Q, Ck, softmax_scale, logp_prev=None, score_kind=SCORE_KL_SHARE):
    logp = np.zeros((s.W, s.Hq, s.Nb, s.K), np.float32)
    D_hi = np.zeros((s.W, s.Hq, s.Nb), np.float32)
    D_i = np.zeros((s.W, s.Nb), np.float32)
    score = np.zeros((s.W, s.K), np.float32)
    _ok(lib().pso_proxy_attn(ctypes.byref(_cshape(s)), dtype, _p(Q), _p(Ck), float(softmax_scale),
                             _p(logp), _p(logp_prev), score_kind, _p(D_hi), _p(D_i), _p(score)),
        "pso_proxy_attn")
    return dict(logp=logp, D_hi=D_hi, D_i=D_i, score=score)


def drift_kl(s: Shape, logp_cur, logp_prev, score_kind=SCORE_KL_SHARE):
    D_hi = np.zeros((s.W, s.Hq, s.Nb), np.float32)
    D_i = np.zeros((s.W, s.Nb), np.float32)
    score = np.zeros((s.W, s.K), np.float32)
    _ok(lib().pso_drift_kl(ctypes.byref(_cshape(s)), _p(logp_cur), _p(logp_prev), score_kind,
                           _p(D_hi), _p(D_i), _p(score)), "pso_drift_kl")
    return dict(D_hi=D_hi, D_i=D_i, score=score)


def topk_clusters(s: Shape, score, k):
    idx = np.zeros((s.W, k), np.int32)
    val = np.zeros((s.W, k), np.float32)
    _ok(lib().pso_topk_clusters(ctypes.byref(_cshape(s)), _p(score), k, _p(idx), _p(val)),
        "pso_topk_clusters")
    return dict(idx=idx, val=val)


def refresh_gather(s: Shape, dtype, assign, idx, k, cap, codes=None, bscale=None, rscale=None,
                   C=None, row_norm=None, want_h=True, Kc=None, Vc=None):
    pos = np.full((s.W, max(cap, 0)), -1, np.int32)
    count = np.zeros((s.W,), np.int32)
    el = _elem(dtype)
    H_hat = np.zeros((s.W, max(cap, 0), s.d), el) if want_h else None
    KV = s.Hkv * s.dh
    K_out = np.zeros((s.W, max(cap, 0), s.Hkv, s.dh), el) if Kc is not None else None
    V_out = np.zeros((s.W, max(cap, 0), s.Hkv, s.dh), el) if Vc is not None else None
    del KV
    _ok(lib().pso_refresh_gather(ctypes.byref(_cshape(s)), dtype, _p(assign), _p(idx), k, cap,
                                 _p(pos), _p(count), _p(codes), _p(bscale), _p(rscale), _p(C),
                                 _p(row_norm), _p(H_hat), _p(Kc), _p(Vc), _p(K_out), _p(V_out)),
        "pso_refresh_gather")
    return dict(pos=pos, count=count, H_hat=H_hat, K_out=K_out, V_out=V_out)


def drift_cosine(s: Shape, C_cur, C_prev):
    """Cosine-dissimilarity drift of every cluster: score [W][K] f32."""
    score = np.zeros((s.W, s.K), np.float32)
    _ok(lib().pso_drift_cosine(ctypes.byref(_cshape(s)), _p(C_cur), _p(C_prev), _p(score)),
        "pso_drift_cosine")
    return score


# ---- Polestar-Commit -------------------------------------------------------
def commit_block(s: Shape, D_i, conf, block_start, alpha, tau_s, hist_sum, hist_n):
    """Current-block commitment.  hist_sum [W][Nb] f64 and hist_n [W] i32 are
    advanced in place; returns commit [W][Nb] u8 (bit 0 drift rule, bit 1
    confidence rule) and delta [W][Nb] f32."""
    assert hist_sum.dtype == np.float64 and hist_n.dtype == np.int32
    commit = np.zeros((s.W, s.Nb), np.uint8)
    delta = np.zeros((s.W, s.Nb), np.float32)
    _ok(lib().pso_commit_block(ctypes.byref(_cshape(s)), _p(D_i), _p(conf), block_start,
                               alpha, tau_s, _p(hist_sum), _p(hist_n), _p(commit), _p(delta)),
        "pso_commit_block")
    return dict(commit=commit, delta=delta)


def commit_suffix(s: Shape, assign, idx, k, block_start, conf, tau_s):
    """Suffix-block commitment: flag [W] u8 and commit [W][N] u8."""
    flag = np.zeros((s.W,), np.uint8)
    commit = np.zeros((s.W, s.N), np.uint8)
    _ok(lib().pso_commit_suffix(ctypes.byref(_cshape(s)), _p(assign), _p(idx), k, block_start,
                                _p(conf), tau_s, _p(flag), _p(commit)), "pso_commit_suffix")
    return dict(flag=flag, commit=commit)
