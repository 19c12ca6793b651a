"""drift_aware_kv_amd -- Python binding of libpolestar_drift.

Polestar-Cache's drift-detection hot path on AMD MI355X (gfx950): spherical
K-Means of the local window, NVFP4 residuals, proxy attention, KL drift, top-k
drifted clusters and the refresh gather; and Polestar-Commit's current-block and
suffix-block commitment rules on that drift.  Every step runs in the HIP kernels of
``libpolestar_drift.so``; this module only marshals arguments (torch tensors ->
device pointers, the current HIP stream) and checks tensor sizes against the
shape before anything is enqueued.  There is no CPU fallback: if the library is
missing, importing the functions raises.

The functions carry the C names (``ps_kmeans_fit`` ...).  Tensors must be
contiguous device tensors; bf16 data is ``torch.bfloat16`` (or ``int16`` /
``uint16`` bit patterns), fp32 data ``torch.float32``.
"""
import ctypes
import os
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpolestar_drift.so")

PS_F32, PS_BF16 = 0, 1
PS_INIT_GIVEN, PS_INIT_STRIDED, PS_INIT_FARTHEST = 0, 1, 2
PS_SCORE_KL_SHARE, PS_SCORE_KL_SHARE_ABS, PS_SCORE_ATTN_WEIGHTED = 0, 1, 2
PS_KMEANS_DEFAULT, PS_KMEANS_FIXED_POINT_EXIT, PS_KMEANS_ALL_PASSES = 0, 1, 2
PS_ERR_SCRATCH_LIMIT = 9
PS_STATIC_SCRATCH_BYTES = 64 << 20     # the library's static K-Means scratch per device

EXPORTS = ("ps_status_string", "ps_workspace_size", "ps_kmeans_fit", "ps_kmeans_fit_static",
           "ps_kmeans_fit_nvfp4", "ps_residual_nvfp4",
           "ps_proxy_attn", "ps_drift_kl", "ps_topk_clusters", "ps_refresh_gather",
           "ps_drift_cosine", "ps_commit_block", "ps_commit_suffix", "ps_profile_begin", "ps_profile_end", "ps_profile_summary")


class PsError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(msg)
        self.status = status


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


_lib = None


def lib():
    """Load the HIP library (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with drift_aware_kv_amd/build.py "
                               "(hipcc, gfx950); there is no CPU fallback")
        L = ctypes.CDLL(LIB_PATH)
        P, I, SP = ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(_CShape)
        L.ps_status_string.argtypes, L.ps_status_string.restype = [I], ctypes.c_char_p
        L.ps_workspace_size.argtypes = [SP, I, ctypes.POINTER(ctypes.c_size_t)]
        L.ps_kmeans_fit.argtypes = [SP, I, P, P, I, ctypes.c_int32, ctypes.c_uint32, P, P, P, P, P,
                                    P, P, ctypes.c_size_t, P]
        L.ps_kmeans_fit_static.argtypes = [SP, I, P, P, I, ctypes.c_int32, ctypes.c_uint32, P, P, P, P,
                                           P, P, P]
        L.ps_kmeans_fit_nvfp4.argtypes = [SP, I, P, P, I, ctypes.c_int32, ctypes.c_uint32, P, P, P, P, P,
                                          P, P, P, P, P, ctypes.c_size_t, P]
        L.ps_residual_nvfp4.argtypes = [SP, I, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.ps_proxy_attn.argtypes = [SP, I, P, P, ctypes.c_float, P, P, I, P, P, P, P]
        L.ps_drift_kl.argtypes = [SP, P, P, I, P, P, P, P]
        L.ps_topk_clusters.argtypes = [SP, P, ctypes.c_int32, P, P, P]
        L.ps_refresh_gather.argtypes = [SP, I, P, P, ctypes.c_int32, ctypes.c_int32, P, P, P, P, P,
                                        P, P, P, P, P, P, P, P]
        F, I32 = ctypes.c_float, ctypes.c_int32
        L.ps_drift_cosine.argtypes = [SP, P, P, P, P]
        L.ps_commit_block.argtypes = [SP, P, P, I32, F, F, P, P, P, P, P]
        L.ps_commit_suffix.argtypes = [SP, P, P, I32, I32, P, F, P, P, P]
        L.ps_profile_begin.argtypes = [ctypes.c_int32]
        L.ps_profile_end.argtypes = []
        L.ps_profile_summary.argtypes = [ctypes.c_char_p, ctypes.c_size_t]
        for n in EXPORTS[1:]:
            getattr(L, n).restype = I
        _lib = L
    return _lib


def profile_begin(max_launches=100000):
    """Start timing every library kernel with HIP events (see the header)."""
    _check(lib().ps_profile_begin(int(max_launches)), "ps_profile_begin")


def profile_end():
    _check(lib().ps_profile_end(), "ps_profile_end")


def profile_summary():
    """{kernel name: (launches, total_ms, min_ms, max_ms, units_done, units)},
    plus '#dropped'.  units is the work of the kernel's launches in the units
    it counts (tiles, rows, clusters) and units_done the part it processed; both
    0 for kernels whose launches always do their full work."""
    buf = ctypes.create_string_buffer(1 << 16)
    _check(lib().ps_profile_summary(buf, len(buf)), "ps_profile_summary")
    out = {}
    for line in buf.value.decode().splitlines():
        f = line.split("\t")
        if f[0] == "#dropped":
            out["#dropped"] = int(f[1])
        elif len(f) == 7:
            out[f[0]] = (int(f[1]), float(f[2]), float(f[3]), float(f[4]), int(f[5]), int(f[6]))
    return out


def status_string(st):
    return lib().ps_status_string(int(st)).decode()


def _check(st, name):
    if st != 0:
        raise PsError(st, f"{name}: {status_string(st)}")


def _cs(s: Shape):
    return ctypes.byref(_CShape(s.W, s.N, s.d, s.Hq, s.Hkv, s.dh, s.Nb, s.K))


_ESIZE = {torch.float32: 4, torch.bfloat16: 2, torch.int16: 2, torch.uint16: 2, torch.int32: 4,
          torch.uint8: 1, torch.float64: 8}


def _ptr(t, numel, esize, name, nullable=False, pinned_ok=False):
    """Device pointer of a contiguous tensor holding at least `numel` elements
    of `esize` bytes (with pinned_ok, pinned host memory is accepted too)."""
    if t is None:
        if nullable:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda and not (pinned_ok and t.is_pinned()):
        raise ValueError(f"{name} must be a device tensor" + (" or pinned host memory" if pinned_ok else ""))
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if _ESIZE.get(t.dtype) != esize:
        raise TypeError(f"{name}: element type {t.dtype} does not match the call ({esize} bytes)")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _es(dtype):
    return 2 if dtype == PS_BF16 else 4


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def ps_workspace_size(s: Shape, dtype) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().ps_workspace_size(_cs(s), dtype, ctypes.byref(n)), "ps_workspace_size")
    return n.value


def workspace(s: Shape, dtype, device=None):
    """Allocate a workspace tensor for ps_kmeans_fit and ps_residual_nvfp4
    (caller-owned)."""
    return torch.empty(max(ps_workspace_size(s, dtype), 16), dtype=torch.uint8, device=device or "cuda")


def ps_kmeans_fit(s: Shape, dtype, H, Kr, init, iters, C, assign, counts, row_norm, Ck=None,
                  objective=None, ws=None, stream=None, flags=0):
    e = _es(dtype)
    KV = s.Hkv * s.dh
    wsb = ps_workspace_size(s, dtype)
    if ws is None:
        raise ValueError("ws is required (see workspace())")
    _check(lib().ps_kmeans_fit(
        _cs(s), dtype, _ptr(H, s.W * s.N * s.d, e, "H"),
        _ptr(Kr, s.W * s.N * KV, e, "Kr", True), init, iters, flags,
        _ptr(C, s.W * s.K * s.d, 4, "C"), _ptr(assign, s.W * s.N, 4, "assign"),
        _ptr(counts, s.W * s.K, 4, "counts"), _ptr(row_norm, s.W * s.N, 4, "row_norm"),
        _ptr(Ck, s.W * s.K * KV, e, "Ck", True), _ptr(objective, s.W, 8, "objective", True),
        _ptr(ws, wsb, 1, "ws"), ws.numel(), _stream(stream)), "ps_kmeans_fit")


def ps_kmeans_fit_static(s: Shape, dtype, H, Kr, init, iters, C, assign, counts, row_norm, Ck=None,
                         objective=None, stream=None, flags=0):
    """ps_kmeans_fit without a workspace: the library's static per-device
    scratch (PS_STATIC_SCRATCH_BYTES) serves instead; nothing is allocated."""
    e = _es(dtype)
    KV = s.Hkv * s.dh
    _check(lib().ps_kmeans_fit_static(
        _cs(s), dtype, _ptr(H, s.W * s.N * s.d, e, "H"),
        _ptr(Kr, s.W * s.N * KV, e, "Kr", True), init, iters, flags,
        _ptr(C, s.W * s.K * s.d, 4, "C"), _ptr(assign, s.W * s.N, 4, "assign"),
        _ptr(counts, s.W * s.K, 4, "counts"), _ptr(row_norm, s.W * s.N, 4, "row_norm"),
        _ptr(Ck, s.W * s.K * KV, e, "Ck", True), _ptr(objective, s.W, 8, "objective", True),
        _stream(stream)), "ps_kmeans_fit_static")


def ps_kmeans_fit_nvfp4(s: Shape, dtype, H, Kr, init, iters, C, assign, counts, row_norm, codes, bscale,
                        rscale, Ck=None, objective=None, ws=None, stream=None, flags=0):
    """ps_kmeans_fit followed by ps_residual_nvfp4 of its outputs, in one call
    (the same results); ws of at least ps_workspace_size bytes."""
    e = _es(dtype)
    KV = s.Hkv * s.dh
    wsb = ps_workspace_size(s, dtype)
    if ws is None:
        raise ValueError("ws is required (see workspace())")
    _check(lib().ps_kmeans_fit_nvfp4(
        _cs(s), dtype, _ptr(H, s.W * s.N * s.d, e, "H"),
        _ptr(Kr, s.W * s.N * KV, e, "Kr", True), init, iters, flags,
        _ptr(C, s.W * s.K * s.d, 4, "C"), _ptr(assign, s.W * s.N, 4, "assign"),
        _ptr(counts, s.W * s.K, 4, "counts"), _ptr(row_norm, s.W * s.N, 4, "row_norm"),
        _ptr(Ck, s.W * s.K * KV, e, "Ck", True), _ptr(objective, s.W, 8, "objective", True),
        _ptr(codes, s.W * s.N * s.d // 2, 1, "codes"), _ptr(bscale, s.W * s.N * s.d // 16, 1, "bscale"),
        _ptr(rscale, s.W * s.N, 4, "rscale"),
        _ptr(ws, wsb, 1, "ws"), ws.numel(), _stream(stream)), "ps_kmeans_fit_nvfp4")


def ps_residual_nvfp4(s: Shape, dtype, H, row_norm, C, assign, codes, bscale, rscale, ws=None,
                      stream=None):
    """ws: optional uint8 scratch tensor of at least 8*W*N + 16 bytes (workspace()
    is always enough): with it, rows are coded grouped by cluster."""
    e = _es(dtype)
    _check(lib().ps_residual_nvfp4(
        _cs(s), dtype, _ptr(H, s.W * s.N * s.d, e, "H"), _ptr(row_norm, s.W * s.N, 4, "row_norm"),
        _ptr(C, s.W * s.K * s.d, 4, "C"), _ptr(assign, s.W * s.N, 4, "assign"),
        _ptr(codes, s.W * s.N * s.d // 2, 1, "codes"), _ptr(bscale, s.W * s.N * s.d // 16, 1, "bscale"),
        _ptr(rscale, s.W * s.N, 4, "rscale"), _ptr(ws, 8 * s.W * s.N + 16, 1, "ws", True),
        ws.numel() if ws is not None else 0, _stream(stream)), "ps_residual_nvfp4")


def ps_proxy_attn(s: Shape, dtype, Q, Ck, softmax_scale, logp_cur, logp_prev, score_kind, D_hi, D_i,
                  score, stream=None):
    e = _es(dtype)
    L = s.W * s.Hq * s.Nb * s.K
    _check(lib().ps_proxy_attn(
        _cs(s), dtype, _ptr(Q, s.W * s.Nb * s.Hq * s.dh, e, "Q"),
        _ptr(Ck, s.W * s.K * s.Hkv * s.dh, e, "Ck"), float(softmax_scale),
        _ptr(logp_cur, L, 4, "logp_cur"), _ptr(logp_prev, L, 4, "logp_prev", True), score_kind,
        _ptr(D_hi, s.W * s.Hq * s.Nb, 4, "D_hi", True), _ptr(D_i, s.W * s.Nb, 4, "D_i"),
        _ptr(score, s.W * s.K, 4, "score"), _stream(stream)), "ps_proxy_attn")


def ps_drift_kl(s: Shape, logp_cur, logp_prev, score_kind, D_hi, D_i, score, stream=None):
    L = s.W * s.Hq * s.Nb * s.K
    _check(lib().ps_drift_kl(
        _cs(s), _ptr(logp_cur, L, 4, "logp_cur"), _ptr(logp_prev, L, 4, "logp_prev"), score_kind,
        _ptr(D_hi, s.W * s.Hq * s.Nb, 4, "D_hi", True), _ptr(D_i, s.W * s.Nb, 4, "D_i"),
        _ptr(score, s.W * s.K, 4, "score"), _stream(stream)), "ps_drift_kl")


def ps_topk_clusters(s: Shape, score, k, idx, val=None, stream=None):
    _check(lib().ps_topk_clusters(
        _cs(s), _ptr(score, s.W * s.K, 4, "score"), int(k), _ptr(idx, s.W * k, 4, "idx"),
        _ptr(val, s.W * k, 4, "val", True), _stream(stream)), "ps_topk_clusters")


def ps_refresh_gather(s: Shape, dtype, assign, idx, k, cap, pos, count, codes=None, bscale=None,
                      rscale=None, C=None, row_norm=None, H_hat=None, Kc=None, Vc=None, K_out=None,
                      V_out=None, stream=None):
    e = _es(dtype)
    KV = s.Hkv * s.dh
    _check(lib().ps_refresh_gather(
        _cs(s), dtype, _ptr(assign, s.W * s.N, 4, "assign"), _ptr(idx, s.W * k, 4, "idx"), int(k),
        int(cap), _ptr(pos, s.W * cap, 4, "pos", cap == 0), _ptr(count, s.W, 4, "count"),
        _ptr(codes, s.W * s.N * s.d // 2, 1, "codes", True, True),
        _ptr(bscale, s.W * s.N * s.d // 16, 1, "bscale", True, True),
        _ptr(rscale, s.W * s.N, 4, "rscale", True, True), _ptr(C, s.W * s.K * s.d, 4, "C", True),
        _ptr(row_norm, s.W * s.N, 4, "row_norm", True),
        _ptr(H_hat, s.W * cap * s.d, e, "H_hat", True), _ptr(Kc, s.W * s.N * KV, e, "Kc", True),
        _ptr(Vc, s.W * s.N * KV, e, "Vc", True), _ptr(K_out, s.W * cap * KV, e, "K_out", True),
        _ptr(V_out, s.W * cap * KV, e, "V_out", True), _stream(stream)), "ps_refresh_gather")


def ps_drift_cosine(s: Shape, C_cur, C_prev, score, stream=None):
    n = s.W * s.K * s.d
    _check(lib().ps_drift_cosine(_cs(s), _ptr(C_cur, n, 4, "C_cur"), _ptr(C_prev, n, 4, "C_prev"),
                                 _ptr(score, s.W * s.K, 4, "score"), _stream(stream)),
           "ps_drift_cosine")


def ps_commit_block(s: Shape, D_i, conf, block_start, alpha, tau_s, hist_sum, hist_n, commit,
                    delta=None, stream=None):
    _check(lib().ps_commit_block(
        _cs(s), _ptr(D_i, s.W * s.Nb, 4, "D_i"), _ptr(conf, s.W * s.N, 4, "conf"),
        int(block_start), float(alpha), float(tau_s), _ptr(hist_sum, s.W * s.Nb, 8, "hist_sum"),
        _ptr(hist_n, s.W, 4, "hist_n"), _ptr(commit, s.W * s.Nb, 1, "commit"),
        _ptr(delta, s.W * s.Nb, 4, "delta", True), _stream(stream)), "ps_commit_block")


def ps_commit_suffix(s: Shape, assign, idx, k, block_start, conf, tau_s, flag, commit, stream=None):
    _check(lib().ps_commit_suffix(
        _cs(s), _ptr(assign, s.W * s.N, 4, "assign"), _ptr(idx, s.W * k, 4, "idx"), int(k),
        int(block_start), _ptr(conf, s.W * s.N, 4, "conf"), float(tau_s),
        _ptr(flag, s.W, 1, "flag"), _ptr(commit, s.W * s.N, 1, "commit"), _stream(stream)),
        "ps_commit_suffix")
