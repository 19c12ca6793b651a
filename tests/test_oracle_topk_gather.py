"""Pins of the oracle's top-k selection and refresh gather against brute force
(numpy's lexsort and set filters) on small inputs with planted ties, NaNs and
capacity overflow."""
import numpy as np
import pytest

import oracle as O


def _brute_topk(s, k):
    idx = np.arange(s.size)
    nan = np.isnan(s)
    key = np.where(nan, 0.0, s)
    key = np.where(key == 0, 0.0, key)          # -0 == +0
    order = np.lexsort((idx, -key, nan))        # NaN last, score desc, index asc
    return order[:k]


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_brute_force(seed):
    rng = np.random.default_rng(30 + seed)
    W, K = 5, int(rng.integers(2, 300))
    s = rng.standard_normal((W, K)).astype(np.float32)
    # planted ties, signed zeros, infinities and NaNs
    s[0, ::3] = 0.5
    s[1, : K // 2] = -0.0
    s[1, K // 2:] = 0.0
    s[2, rng.integers(0, K, 4)] = np.nan
    s[3, 0] = np.inf
    s[3, -1] = -np.inf
    s[4, :] = np.nan
    k = int(rng.integers(1, K + 1))
    shp = O.Shape(W=W, N=K, d=16, K=K)
    r = O.topk_clusters(shp, s, k)
    for w in range(W):
        ref = _brute_topk(s[w], k)
        assert np.array_equal(r["idx"][w], ref), (w, r["idx"][w], ref)
        assert np.array_equal(r["val"][w], s[w][ref], equal_nan=True)
        sel = set(ref.tolist())
        rest = [i for i in range(K) if i not in sel]
        fin = ~np.isnan(s[w][ref])
        if rest and fin.any():
            lo = s[w][ref][fin].min()
            others = s[w][rest]
            assert np.all(others[~np.isnan(others)] <= lo)


def test_topk_range_errors():
    shp = O.Shape(W=1, N=4, d=16, K=4)
    with pytest.raises(O.OracleError):
        O.topk_clusters(shp, np.zeros((1, 4), np.float32), 5)
    with pytest.raises(O.OracleError):
        O.topk_clusters(shp, np.zeros((1, 4), np.float32), 0)


def _codes_for(rng, W, N, d, K):
    H = rng.standard_normal((W, N, d)).astype(np.float32)
    C = rng.standard_normal((W, K, d)).astype(np.float32)
    C /= np.linalg.norm(C, axis=-1, keepdims=True)
    assign = rng.integers(0, K, size=(W, N)).astype(np.int32)
    rn = np.linalg.norm(H.astype(np.float64), axis=-1).astype(np.float32)
    s = O.Shape(W=W, N=N, d=d, K=K)
    q = O.residual_nvfp4(s, O.F32, H, rn, C, assign)
    return H, C, assign, rn, q


@pytest.mark.parametrize("cap_mode", ["ample", "exact", "short", "zero"])
def test_gather_matches_set_filter(cap_mode):
    rng = np.random.default_rng(40)
    W, N, d, K, k, Hkv, dh = 3, 97, 64, 7, 3, 2, 8
    H, C, assign, rn, q = _codes_for(rng, W, N, d, K)
    idx = np.stack([rng.choice(K, size=k, replace=False) for _ in range(W)]).astype(np.int32)
    Kc = rng.standard_normal((W, N, Hkv, dh)).astype(np.float32)
    Vc = rng.standard_normal((W, N, Hkv, dh)).astype(np.float32)
    true = [np.nonzero(np.isin(assign[w], idx[w]))[0] for w in range(W)]
    cap = {"ample": N, "exact": max(len(t) for t in true), "short": 5, "zero": 0}[cap_mode]
    s = O.Shape(W=W, N=N, d=d, Hq=2, Hkv=Hkv, dh=dh, K=K)
    r = O.refresh_gather(s, O.F32, assign, idx, k, cap, q["codes"], q["bscale"], q["rscale"],
                         C, rn, True, Kc, Vc)
    for w in range(W):
        t = true[w]
        assert r["count"][w] == t.size
        counts = np.bincount(assign[w], minlength=K)
        assert r["count"][w] == counts[idx[w]].sum()
        m = min(t.size, cap)
        assert np.array_equal(r["pos"][w, :m], t[:m])
        assert np.all(r["pos"][w, m:] == -1)            # untouched slots
        assert np.array_equal(r["K_out"][w, :m], Kc[w, t[:m]])
        assert np.array_equal(r["V_out"][w, :m], Vc[w, t[:m]])
        # reconstruction lands within the NVFP4 bound of the original row:
        # |h - hhat| <= n * eff * 1 per element (coarsest E2M1 half-spacing)
        for slot in range(m):
            j = t[slot]
            sdec = np.array([O.e4m3_decode(c) for c in q["bscale"][w, j]], np.float64)
            eff = np.repeat(sdec, 16) * float(q["rscale"][w, j])
            err = np.abs(r["H_hat"][w, slot].astype(np.float64) - H[w, j].astype(np.float64))
            assert np.all(err <= rn[w, j] * (eff * 1.0 + 1e-6) + 1e-6)


def test_gather_bf16_rows_are_byte_copies():
    rng = np.random.default_rng(41)
    W, N, d, K, k = 1, 32, 16, 4, 1
    assign = (np.arange(N) % K).astype(np.int32)[None]
    idx = np.array([[2]], np.int32)
    Kc = rng.integers(0, 65535, size=(W, N, 1, 16)).astype(np.uint16)
    Kc[0, 2, 0, 0] = 0x7F81  # a signalling NaN pattern must survive
    s = O.Shape(W=W, N=N, d=d, Hq=1, Hkv=1, dh=16, K=K)
    r = O.refresh_gather(s, O.BF16, assign, idx, k, N, want_h=False, Kc=Kc, Vc=Kc)
    t = np.arange(2, N, K)
    assert r["count"][0] == t.size
    assert np.array_equal(r["K_out"][0, : t.size], Kc[0, t])


def test_gather_rebuilds_representable_rows_exactly():
    """Rows built from NVFP4-representable residuals (centre 0, every block
    holding a +-6, power-of-two row scale) times a power-of-two norm n are
    rebuilt exactly: h_hat = (c + rhat) * n == h, bit for bit."""
    rng = np.random.default_rng(8)
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    N, d, K = 24, 64, 2
    nb = d // 16
    nib = rng.integers(0, 16, size=(N, d)).astype(np.uint8)
    nib[nib == 8] = 0
    for j in range(N):
        for b in range(nb):
            nib[j, 16 * b + rng.integers(0, 16)] = 7 | (8 * rng.integers(0, 2))
    sc = rng.integers(0x08, 0x7E, size=(N, nb)).astype(np.uint8)
    sc[np.arange(N), rng.integers(0, nb, size=N)] = 0x7E
    g = np.ldexp(1.0, rng.integers(-20, -6, size=N))
    sval = np.array([[O.e4m3_decode(c) for c in row] for row in sc])
    x = np.where(nib & 8, -1.0, 1.0) * mags[nib & 7] * np.repeat(sval, 16, axis=1) * g[:, None]
    n = np.ldexp(1.0, rng.integers(-3, 9, size=N)).astype(np.float32)     # powers of two, not 1
    H = (x * n[:, None]).astype(np.float32)[None]
    s = O.Shape(W=1, N=N, d=d, K=K)
    C = np.zeros((1, K, d), np.float32)
    assign = np.zeros((1, N), np.int32)
    rn = n[None].copy()
    q = O.residual_nvfp4(s, O.F32, H, rn, C, assign)
    idx = np.array([[0, 1]], np.int32)
    r = O.refresh_gather(s, O.F32, assign, idx, 2, N, q["codes"], q["bscale"], q["rscale"], C, rn, True)
    assert int(r["count"][0]) == N
    assert np.array_equal(r["H_hat"][0].view(np.uint32), H[0].view(np.uint32))
