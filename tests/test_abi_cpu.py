"""CPU-side checks of the C ABI: the HIP library loads, exports every entry
point that include/*.h declares, and rejects bad host-known arguments with the
documented status codes before anything is enqueued (no GPU is touched: every
case here fails validation, so no kernel launch is attempted)."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBPATH = os.path.join(ROOT, "drift_aware_kv_amd", "libpolestar_drift.so")

OK, NULL, SHAPE, DTYPE, ALIGN, RANGE, WORKSPACE, DEVICE, MEMORY, SCRATCH_LIMIT = range(10)


def declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+char\s*\*|ps_status)\s+(ps_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(LIBPATH):
        import drift_aware_kv_amd.build as b
        b.build()
    import drift_aware_kv_amd as P
    return P.lib()


def test_header_declares_the_six_calls():
    names = declared_functions()
    for n in ("ps_kmeans_fit", "ps_residual_nvfp4", "ps_proxy_attn", "ps_drift_kl",
              "ps_topk_clusters", "ps_refresh_gather", "ps_status_string", "ps_workspace_size"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    raw = ctypes.CDLL(LIBPATH)
    for n in declared_functions():
        assert hasattr(raw, n), n


def test_status_strings(L):
    import drift_aware_kv_amd as P
    for st in range(10):
        assert P.status_string(st).startswith("PS_")
    assert "unknown" in P.status_string(99)


def _shape(**kw):
    import drift_aware_kv_amd as P
    base = dict(W=2, N=64, d=32, Hq=4, Hkv=2, dh=16, Nb=8, K=4)
    base.update(kw)
    return P._CShape(*[base[k] for k in ("W", "N", "d", "Hq", "Hkv", "dh", "Nb", "K")])


FAKE = ctypes.c_void_p(0x10000)       # aligned, never dereferenced in these cases
MISALIGNED = ctypes.c_void_p(0x10004)


def test_workspace_size(L):
    n = ctypes.c_size_t(0)
    assert L.ps_workspace_size(ctypes.byref(_shape()), 1, ctypes.byref(n)) == OK
    bf = n.value
    assert bf >= 2 * 4 * 32 * 2 + 2 * 64 * 4  # bf16 centres + member lists
    assert L.ps_workspace_size(ctypes.byref(_shape()), 0, ctypes.byref(n)) == OK
    assert n.value < bf                        # the fp32 path keeps no bf16 copy
    assert L.ps_workspace_size(ctypes.byref(_shape(K=65)), 1, ctypes.byref(n)) == SHAPE
    assert L.ps_workspace_size(ctypes.byref(_shape()), 7, ctypes.byref(n)) == DTYPE
    assert L.ps_workspace_size(None, 1, ctypes.byref(n)) == NULL
    # the same scratch also serves the NVFP4 coder (8 W N + 16 bytes), also on
    # shapes whose K-Means needs are smaller than that
    for kw in (dict(W=3, N=4000, d=16, K=1), dict(W=1, N=64, d=32, K=4), dict(W=7, N=300, d=4096, K=64)):
        for dt in (0, 1):
            assert L.ps_workspace_size(ctypes.byref(_shape(**kw)), dt, ctypes.byref(n)) == OK
            assert n.value >= 8 * kw["W"] * kw["N"] + 16, (kw, dt, n.value)


def _fit(L, shape, dtype=1, init=1, iters=2, H=FAKE, ws=FAKE, ws_bytes=1 << 30, C=FAKE, Kr=None,
         Ck=None, flags=0):
    return L.ps_kmeans_fit(ctypes.byref(shape), dtype, H, Kr, init, iters, flags, C, FAKE, FAKE, FAKE,
                           Ck, None, ws, ws_bytes, None)


def test_kmeans_fit_argument_checks(L):
    s = _shape()
    assert _fit(L, s, H=None) == NULL
    assert _fit(L, s, C=None) == NULL
    assert _fit(L, s, Kr=FAKE, Ck=None) == NULL           # Kr and Ck come together
    assert _fit(L, s, dtype=3) == DTYPE
    assert _fit(L, _shape(d=24)) == SHAPE                   # d % 16
    assert _fit(L, _shape(d=8208)) == SHAPE                 # d > 8192
    assert _fit(L, _shape(K=65)) == SHAPE                   # K > N
    assert _fit(L, _shape(K=0)) == SHAPE
    assert _fit(L, _shape(Hq=3, Hkv=2), Kr=FAKE, Ck=FAKE) == SHAPE   # Hq % Hkv
    assert _fit(L, _shape(dh=12), Kr=FAKE, Ck=FAKE) == SHAPE         # dh % 8
    assert _fit(L, s, iters=0) == RANGE
    assert _fit(L, s, init=9) == RANGE
    assert _fit(L, s, flags=4) == RANGE                     # unknown flag bit
    assert _fit(L, s, flags=3) == RANGE                     # fixed-point exit and all passes at once
    assert _fit(L, s, H=MISALIGNED) == ALIGN
    assert _fit(L, s, ws=None) == WORKSPACE
    assert _fit(L, s, ws_bytes=16) == WORKSPACE
    # W = 0 is a valid no-op and enqueues nothing
    assert _fit(L, _shape(W=0)) == OK


def _fit_code(L, shape, dtype=1, H=FAKE, iters=2, codes=FAKE, bscale=FAKE, rscale=FAKE, ws=FAKE,
              ws_bytes=1 << 30, flags=0):
    return L.ps_kmeans_fit_nvfp4(ctypes.byref(shape), dtype, H, None, 1, iters, flags, FAKE, FAKE, FAKE, FAKE,
                                 None, None, codes, bscale, rscale, ws, ws_bytes, None)


def test_kmeans_fit_nvfp4_argument_checks(L):
    """The fit-and-code call checks the K-Means arguments, then the coder's
    outputs, then the workspace (ps_workspace_size covers both calls)."""
    s = _shape()
    assert _fit_code(L, s, H=None) == NULL
    assert _fit_code(L, s, iters=0) == RANGE
    assert _fit_code(L, _shape(K=65)) == SHAPE
    assert _fit_code(L, s, codes=None) == NULL
    assert _fit_code(L, s, bscale=None) == NULL
    assert _fit_code(L, s, rscale=None) == NULL
    assert _fit_code(L, s, rscale=MISALIGNED) == ALIGN
    assert _fit_code(L, s, ws=None) == WORKSPACE
    for kw in (dict(), dict(W=3, N=4000, d=16, K=1), dict(W=2, N=300, d=4096, K=64), dict(d=8192)):
        for dt in (0, 1):
            sh = _shape(**kw)
            n = ctypes.c_size_t(0)
            assert L.ps_workspace_size(ctypes.byref(sh), dt, ctypes.byref(n)) == OK
            assert _fit_code(L, sh, dtype=dt, ws_bytes=n.value - 1) == WORKSPACE, (kw, dt)
    assert _fit_code(L, _shape(W=0)) == OK          # nothing to do: no device touched


def _fit_static(L, shape, dtype=1, H=FAKE, Kr=None, init=1, iters=2, C=FAKE, Ck=None, flags=0):
    return L.ps_kmeans_fit_static(ctypes.byref(shape), dtype, H, Kr, init, iters, flags, C, FAKE, FAKE, FAKE,
                                  Ck, None, None)


def test_kmeans_fit_static_argument_checks(L):
    """The allocation-free variant checks the same arguments before it looks
    up its scratch, and refuses a shape whose K-Means scratch exceeds the
    static array (512 windows of 1024 x 4096 with 64 clusters need 256 MiB of
    bf16 centres alone)."""
    import drift_aware_kv_amd as P
    s = _shape()
    assert _fit_static(L, s, H=None) == NULL
    assert _fit_static(L, s, Kr=FAKE, Ck=None) == NULL
    assert _fit_static(L, s, dtype=3) == DTYPE
    assert _fit_static(L, _shape(K=65)) == SHAPE
    assert _fit_static(L, s, iters=0) == RANGE
    assert _fit_static(L, s, H=MISALIGNED) == ALIGN
    big = _shape(W=512, N=1024, d=4096, K=64)
    assert _fit_static(L, big) == SCRATCH_LIMIT
    n = ctypes.c_size_t(0)
    assert L.ps_workspace_size(ctypes.byref(big), 1, ctypes.byref(n)) == OK
    assert n.value > P.PS_STATIC_SCRATCH_BYTES
    assert "static scratch" in P.status_string(SCRATCH_LIMIT)
    assert _fit_static(L, _shape(W=0)) == OK       # nothing to do: no device touched


def test_residual_argument_checks(L):
    s = _shape()
    f = lambda s=s, dt=1, H=FAKE, ws=None, wsb=0: L.ps_residual_nvfp4(
        ctypes.byref(s), dt, H, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, wsb, None)
    assert f(H=None) == NULL
    assert f(dt=5) == DTYPE
    assert f(s=_shape(d=8)) == SHAPE
    assert f(s=_shape(d=8208)) == SHAPE                      # d > 8192
    assert f(H=MISALIGNED) == ALIGN
    assert f(ws=MISALIGNED, wsb=1 << 20) == ALIGN
    assert f(ws=FAKE, wsb=8 * 2 * 64 + 15) == WORKSPACE    # needs 8 * W * N + 16 bytes
    assert f(s=_shape(W=0)) == OK
    assert f(s=_shape(W=0), ws=FAKE, wsb=16) == OK


def test_proxy_and_drift_argument_checks(L):
    s = _shape()
    f = lambda s=s, Q=FAKE, prev=FAKE, kind=0, cur=FAKE: L.ps_proxy_attn(
        ctypes.byref(s), 1, Q, FAKE, ctypes.c_float(0.25), cur, prev, kind, None, FAKE, FAKE, None)
    assert f(Q=None) == NULL
    assert f(kind=3) == RANGE
    assert f(prev=FAKE, cur=FAKE) == RANGE                 # logp_prev aliases logp_cur
    assert f(s=_shape(Hq=3)) == SHAPE
    assert f(s=_shape(Nb=65)) == SHAPE
    assert f(s=_shape(Hq=256, Hkv=256, Nb=64)) == SHAPE       # Hq * Nb + 4 K > 16384
    assert f(s=_shape(W=0), prev=None) == OK
    g = lambda s=s, kind=0: L.ps_drift_kl(ctypes.byref(s), FAKE, ctypes.c_void_p(0x20000), kind, None,
                                          FAKE, FAKE, None)
    assert g(kind=-1) == RANGE
    assert g(s=_shape(K=2000)) == SHAPE
    assert g(s=_shape(W=0)) == OK


def test_topk_and_gather_argument_checks(L):
    s = _shape()
    t = lambda k, s=s: L.ps_topk_clusters(ctypes.byref(s), FAKE, k, FAKE, None, None)
    assert t(0) == RANGE
    assert t(5) == RANGE                                   # k > K
    assert t(4, s=_shape(W=0)) == OK
    g = lambda k=2, cap=8, pos=FAKE, Hh=None, codes=None: L.ps_refresh_gather(
        ctypes.byref(s), 1, FAKE, FAKE, k, cap, pos, FAKE, codes, None, None, None, None, Hh, None,
        None, None, None, None)
    assert g(k=0) == RANGE
    assert g(cap=-1) == RANGE
    assert g(pos=None) == NULL                             # cap > 0 needs pos
    assert g(Hh=FAKE) == NULL                              # H_hat needs the residual inputs
    assert L.ps_refresh_gather(ctypes.byref(_shape(W=0)), 1, FAKE, FAKE, 2, 0, None, FAKE, None,
                               None, None, None, None, None, None, None, None, None, None) == OK
    # a residual store at an address that is neither device memory nor
    # device-mapped pinned host memory is refused before any launch
    host_buf = ctypes.create_string_buffer(1 << 12)
    hb = ctypes.c_void_p((ctypes.addressof(host_buf) + 15) & ~15)
    assert L.ps_refresh_gather(ctypes.byref(s), 1, FAKE, FAKE, 2, 8, FAKE, FAKE, hb, hb, hb, FAKE,
                               FAKE, FAKE, None, None, None, None, None) == MEMORY


def test_commit_argument_checks(L):
    s = _shape()                                           # N=64, Nb=8, K=4
    b = lambda s=s, b0=10, alpha=1.0, tau=0.9, D=FAKE, delta=None: L.ps_commit_block(
        ctypes.byref(s), D, FAKE, b0, alpha, tau, FAKE, FAKE, FAKE, delta, None)
    assert b(D=None) == NULL
    assert b(b0=-1) == RANGE
    assert b(b0=57) == RANGE                               # block past the window end
    assert b(alpha=-0.5) == RANGE
    assert b(alpha=float("nan")) == RANGE
    assert b(tau=float("inf")) == RANGE
    assert b(D=MISALIGNED) == ALIGN
    assert b(delta=MISALIGNED) == ALIGN
    assert b(s=_shape(Nb=65)) == SHAPE
    assert b(s=_shape(W=0)) == OK
    assert b(s=_shape(W=0), b0=56) == OK                   # last valid block start
    u = lambda s=s, k=2, b0=10, tau=0.9, flag=FAKE: L.ps_commit_suffix(
        ctypes.byref(s), FAKE, FAKE, k, b0, FAKE, tau, flag, FAKE, None)
    assert u(flag=None) == NULL
    assert u(k=0) == RANGE
    assert u(k=5) == RANGE                                 # k > K
    assert u(b0=60) == RANGE
    assert u(tau=float("nan")) == RANGE
    assert u(flag=MISALIGNED) == ALIGN
    assert u(s=_shape(K=2000)) == SHAPE
    assert u(s=_shape(W=0)) == OK


def test_drift_cosine_argument_checks(L):
    c = lambda s=_shape(), a=FAKE, sc=FAKE: L.ps_drift_cosine(ctypes.byref(s), a, FAKE, sc, None)
    assert c(a=None) == NULL
    assert c(s=_shape(d=24)) == SHAPE                      # d % 16 != 0
    assert c(s=_shape(K=0)) == SHAPE
    assert c(sc=MISALIGNED) == ALIGN
    assert c(s=_shape(W=0)) == OK
