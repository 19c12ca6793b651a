"""GPU parity of each library call against the oracle.  Both sides get the
same seeded host-generated inputs; the oracle never reads anything the device
computed (chained calls chain each side on its own results).  Integer and byte results are bit-exact except
documented near-ties; floating-point results within 1e-3 relative / 1e-5
absolute.  Shapes span several tiles with ragged tails (N not a multiple of
128, K not a multiple of 16, d not a multiple of 64, dh not a multiple of 32)."""
import sys
import zlib

import numpy as np
import pytest
import torch

import oracle as O
from parity_helpers import (assignment_mismatches, bf16f, check_centre_properties, close, dev, host,
                            max_rel)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import drift_aware_kv_amd as P
    P.lib()
    return P


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def rnd_bf16(rng, shape, scale=1.0):
    return O.f32_to_bf16((rng.standard_normal(shape) * scale).astype(np.float32)) if np.prod(shape) < 4e6 \
        else _fast_bf16(rng, shape, scale)


def _fast_bf16(rng, shape, scale):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    u = x.view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


KM_CASES = [
    # name, W, N, d, K, Hkv, dh, bf16
    ("ragged-bf16", 3, 300, 80, 37, 2, 24, True),
    ("k300-two-groups", 1, 600, 64, 300, 1, 32, True),
    ("tiny-f32", 2, 200, 64, 8, 1, 64, False),
    ("llada-row", 1, 256, 4096, 64, 32, 128, True),
    ("dream-rows", 1, 512, 3584, 128, 4, 128, True),   # d not a multiple of 2048
    ("k1", 2, 130, 48, 1, 1, 16, True),
    ("k256-llada-rows", 2, 700, 4096, 256, 8, 128, True),   # the 256-cluster tile kernel (LDS-fed)
    ("k1000-four-groups", 1, 1100, 192, 1000, 2, 32, True),  # four cluster groups, ragged
    ("k200-d80", 2, 400, 80, 200, 1, 16, True),   # d not a multiple of 32: the register-staged tile kernel
    ("d8192", 1, 300, 8192, 70, 2, 64, True),     # the longest rows the update accepts
    ("k200-d8192", 1, 400, 8192, 200, 2, 64, True),
]


@pytest.mark.parametrize("case", KM_CASES, ids=[c[0] for c in KM_CASES])
def test_kmeans_iterations(P, case):
    """Four Lloyd iterations, one call each, on both sides (STRIDED first,
    then GIVEN).  Every iteration must give the same assignment, counts,
    centres, keys and objective.  A row assigned differently must be a
    near-tie under the centres both sides started the iteration from; the
    clusters such rows touch are then left out of that iteration's
    comparison, and the device restarts the next iteration from the oracle's
    centres and keys, so every iteration is compared on every other cluster.
    The data of each case come from a fixed seed (crc32 of its name)."""
    name, W, N, d, K, Hkv, dh, bf = case
    say("kmeans iterations", name)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    dt = P.PS_BF16 if bf else P.PS_F32
    H = rnd_bf16(rng, (W, N, d)) if bf else rng.standard_normal((W, N, d)).astype(np.float32)
    Kr = rnd_bf16(rng, (W, N, Hkv, dh)) if bf else rng.standard_normal((W, N, Hkv, dh)).astype(np.float32)
    s = P.Shape(W=W, N=N, d=d, Hq=Hkv, Hkv=Hkv, dh=dh, Nb=1, K=K)
    so = O.Shape(W=W, N=N, d=d, Hq=Hkv, Hkv=Hkv, dh=dh, Nb=1, K=K)
    Hd, Krd = dev(H), dev(Kr)
    C = torch.zeros(W, K, d, dtype=torch.float32, device="cuda")
    a = torch.zeros(W, N, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(W, K, dtype=torch.int32, device="cuda")
    rn = torch.zeros(W, N, dtype=torch.float32, device="cuda")
    Ck = torch.zeros(W, K, Hkv, dh, dtype=torch.bfloat16 if bf else torch.float32, device="cuda")
    obj = torch.zeros(W, dtype=torch.float64, device="cuda")
    ws = P.workspace(s, dt)
    odt = O.BF16 if bf else O.F32
    oC = np.zeros((W, K, d), np.float32)                       # the oracle's own chain
    oCk = np.zeros((W, K, Hkv, dh), np.uint16 if bf else np.float32)
    full = 0
    for it in range(4):
        init = P.PS_INIT_STRIDED if it == 0 else P.PS_INIT_GIVEN
        C_in = O.kmeans_init(so, odt, H, O.INIT_STRIDED) if it == 0 else oC.copy()
        P.ps_kmeans_fit(s, dt, Hd, Krd, init, 1, C, a, cnt, rn, Ck, obj, ws)
        torch.cuda.synchronize()
        r = O.kmeans_fit(so, odt, H, Kr, O.INIT_STRIDED if it == 0 else O.INIT_GIVEN, 1, oC.copy(),
                         oCk.copy())
        ga, gC, gn, gcnt, gCk, gobj = host(a), host(C), host(rn), host(cnt), host(Ck), host(obj)
        assert max_rel(gn, r["row_norm"]) <= 1.2e-7, "row norms"
        for w in range(W):
            check_centre_properties(H[w], bf, gn[w], ga[w], gC[w], gcnt[w])
        keep = np.ones((W, K), bool)       # clusters no near-tie row touches
        n_ties = 0
        for w in range(W):
            t_w, real = assignment_mismatches(H[w], C_in[w], bf, ga[w], r["assign"][w],
                                              r["row_norm"][w])
            assert not real, f"iter {it} window {w}: {len(real)} assignment disagreements"
            keep[w, ga[w][t_w]] = False
            keep[w, r["assign"][w][t_w]] = False
            n_ties += len(t_w)
        assert np.array_equal(gcnt[keep], r["counts"][keep])
        assert close(gC[keep], r["C"][keep], 1e-6, 1e-7), f"centres iter {it}: {max_rel(gC, r['C'])}"
        if bf:
            assert np.array_equal(gCk[keep], r["Ck"][keep]), "centroid keys"
        else:
            assert close(gCk[keep], r["Ck"][keep], 1e-6, 1e-7)
        if n_ties:
            say(f"  iteration {it}: {n_ties} near-tie rows; {int((~keep).sum())} clusters left out, "
                "the device restarts from the oracle's centres")
            C.copy_(dev(r["C"]))
            Ck.copy_(dev(r["Ck"]).view(Ck.dtype) if bf else dev(r["Ck"]))
        else:
            assert close(gobj, r["objective"], 1e-9, 1e-9)
            full += 1
        oC, oCk = r["C"], r["Ck"]
    say(f"  {full} of 4 iterations compared on every cluster")


ITER_CASES = [("ragged-bf16", 3, 300, 80, 37, True), ("llada-rows", 2, 1024, 4096, 64, True),
              ("f32", 2, 256, 64, 8, False),
              # above 128 clusters: passes after the first run the LDS-fed tile
              # kernel, a single pass the register-staged one (same score order)
              ("k256-llada-rows", 2, 700, 4096, 256, True),
              ("k300-two-groups-ragged", 1, 640, 192, 300, True),
              ("k150-one-chunk", 2, 300, 64, 150, True),
              ("k200-d96", 1, 500, 96, 200, True),   # d not a multiple of 64: register-staged passes
              ("k200-d8192", 1, 400, 8192, 200, True),
              # 16384 clusters in the batch: the later updates take four per workgroup
              ("k256-w64", 64, 512, 128, 256, True)]


@pytest.mark.parametrize("case", ITER_CASES, ids=[c[0] for c in ITER_CASES])
def test_iteration_paths_agree(P, case):
    """One call of n iterations with every pass in full (later iterations
    re-sum only the clusters whose members changed), n calls of one iteration
    (every cluster re-summed each time), and n iterations with the default
    fixed-point exit (a window's passes stop once one moves no row) must give
    bit-identical centres, assignments, counts, keys and objective."""
    name, W, N, d, K, bf = case
    say("iteration paths", name)
    rng = np.random.default_rng(21)
    dt = P.PS_BF16 if bf else P.PS_F32
    H = rnd_bf16(rng, (W, N, d)) if bf else rng.standard_normal((W, N, d)).astype(np.float32)
    Kr = rnd_bf16(rng, (W, N, 2, 16)) if bf else rng.standard_normal((W, N, 2, 16)).astype(np.float32)
    s = P.Shape(W=W, N=N, d=d, Hq=2, Hkv=2, dh=16, Nb=1, K=K)
    Hd, Krd = dev(H), dev(Kr)
    et = torch.bfloat16 if bf else torch.float32
    n = 6

    def fresh():
        return dict(C=torch.zeros(W, K, d, device="cuda"),
                    a=torch.zeros(W, N, dtype=torch.int32, device="cuda"),
                    cnt=torch.zeros(W, K, dtype=torch.int32, device="cuda"),
                    rn=torch.zeros(W, N, device="cuda"), Ck=torch.zeros(W, K, 2, 16, dtype=et, device="cuda"),
                    obj=torch.zeros(W, dtype=torch.float64, device="cuda"), ws=P.workspace(s, dt))

    def run(st, init, iters, flags):
        P.ps_kmeans_fit(s, dt, Hd, Krd, init, iters, st["C"], st["a"], st["cnt"], st["rn"], st["Ck"],
                        st["obj"], st["ws"], flags=flags)

    A, B, X = fresh(), fresh(), fresh()
    run(A, P.PS_INIT_STRIDED, n, P.PS_KMEANS_ALL_PASSES)
    run(B, P.PS_INIT_STRIDED, 1, P.PS_KMEANS_ALL_PASSES)
    for _ in range(n - 1):
        run(B, P.PS_INIT_GIVEN, 1, P.PS_KMEANS_ALL_PASSES)
    run(X, P.PS_INIT_STRIDED, n, P.PS_KMEANS_DEFAULT)      # windows stop at their fixed point
    torch.cuda.synchronize()
    for key in ("C", "a", "cnt", "Ck", "obj", "rn"):
        a, b, x = host(A[key]), host(B[key]), host(X[key])
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), key
        assert np.array_equal(a.view(np.uint8), x.view(np.uint8)), key


@pytest.mark.parametrize("K", [64, 128])
def test_assign_tile_width_does_not_change_results(P, K):
    """Launches with fewer token tiles than compute units give each wave one
    16-token block instead of several: 80 windows in one call (several
    blocks per wave) and the same windows one at a time (one block) must give
    bit-identical centres, assignments, counts, norms, keys and objective."""
    rng = np.random.default_rng(K)
    W, N, d, Hkv, dh = 80, 1024, 64, 1, 16
    H = rnd_bf16(rng, (W, N, d))
    Kr = rnd_bf16(rng, (W, N, Hkv, dh))

    def fit(h, kr):
        Wc = h.shape[0]
        s = P.Shape(W=Wc, N=N, d=d, Hq=Hkv, Hkv=Hkv, dh=dh, Nb=1, K=K)
        out = dict(C=torch.zeros(Wc, K, d, device="cuda"), a=torch.zeros(Wc, N, dtype=torch.int32, device="cuda"),
                   cnt=torch.zeros(Wc, K, dtype=torch.int32, device="cuda"), rn=torch.zeros(Wc, N, device="cuda"),
                   Ck=torch.zeros(Wc, K, Hkv, dh, dtype=torch.bfloat16, device="cuda"),
                   obj=torch.zeros(Wc, dtype=torch.float64, device="cuda"))
        P.ps_kmeans_fit(s, P.PS_BF16, dev(h), dev(kr), P.PS_INIT_STRIDED, 4, out["C"], out["a"], out["cnt"],
                        out["rn"], out["Ck"], out["obj"], P.workspace(s, P.PS_BF16))
        torch.cuda.synchronize()
        return {k: host(v) for k, v in out.items()}

    batch = fit(H, Kr)
    for w in (0, 37, 79):
        say("window", w, "alone, K =", K)
        alone = fit(H[w:w + 1], Kr[w:w + 1])
        for key, v in alone.items():
            assert np.array_equal(batch[key][w:w + 1].view(np.uint8), v.view(np.uint8)), (w, key)


def test_kmeans_chained_planted_exact(P):
    """The tiny planted case, chained end to end from FARTHEST seeding over 10
    iterations, must equal the oracle exactly."""
    import synth
    cfg = synth.CONFIGS["tiny-planted"]
    data = synth.generate(cfg)
    s = P.Shape(W=1, N=cfg.N, d=cfg.d, Hq=1, Hkv=1, dh=cfg.dh, Nb=cfg.Nb, K=cfg.K)
    so = O.Shape(W=1, N=cfg.N, d=cfg.d, Hq=1, Hkv=1, dh=cfg.dh, Nb=cfg.Nb, K=cfg.K)
    C = torch.zeros(1, cfg.K, cfg.d, device="cuda")
    a = torch.zeros(1, cfg.N, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(1, cfg.K, dtype=torch.int32, device="cuda")
    rn = torch.zeros(1, cfg.N, device="cuda")
    Ck = torch.zeros(1, cfg.K, 1, cfg.dh, device="cuda")
    obj = torch.zeros(1, dtype=torch.float64, device="cuda")
    P.ps_kmeans_fit(s, P.PS_F32, dev(data["H"]), dev(data["Kr"]), P.PS_INIT_FARTHEST, cfg.iters, C, a,
                    cnt, rn, Ck, obj, P.workspace(s, P.PS_F32))
    torch.cuda.synchronize()
    r = O.kmeans_fit(so, O.F32, data["H"], data["Kr"], O.INIT_FARTHEST, cfg.iters,
                     np.zeros((1, cfg.K, cfg.d), np.float32))
    assert np.array_equal(host(a), r["assign"])
    assert np.array_equal(host(cnt), r["counts"])
    assert close(host(C), r["C"], 1e-6, 1e-7)
    assert close(host(Ck), r["Ck"], 1e-6, 1e-7)
    assert max_rel(host(rn), r["row_norm"]) <= 1.2e-7


@pytest.mark.parametrize("bf", [True, False])
def test_farthest_seeding_matches(P, bf):
    rng = np.random.default_rng(5)
    W, N, d, K = 2, 333, 96, 11
    H = rnd_bf16(rng, (W, N, d)) if bf else rng.standard_normal((W, N, d)).astype(np.float32)
    H[0, 7] = 0  # a zero row is never a seed
    dt = P.PS_BF16 if bf else P.PS_F32
    s = P.Shape(W=W, N=N, d=d, K=K)
    C = torch.zeros(W, K, d, device="cuda")
    a = torch.zeros(W, N, dtype=torch.int32, device="cuda")
    P.ps_kmeans_fit(s, dt, dev(H), None, P.PS_INIT_FARTHEST, 1, C, a,
                    torch.zeros(W, K, dtype=torch.int32, device="cuda"),
                    torch.zeros(W, N, device="cuda"), None, None, P.workspace(s, dt))
    torch.cuda.synchronize()
    seeds = O.kmeans_init(O.Shape(W=W, N=N, d=d, K=K), O.BF16 if bf else O.F32, H, O.INIT_FARTHEST)
    r = O.kmeans_fit(O.Shape(W=W, N=N, d=d, K=K), O.BF16 if bf else O.F32, H, None, O.INIT_GIVEN, 1,
                     seeds.copy())
    assert np.array_equal(host(a), r["assign"])
    assert close(host(C), r["C"], 1e-6, 1e-7)


# hidden sizes covering every thread layout of the coder, full and ragged:
# one wave with 1, 2 or 4 blocks of 16 per thread, four waves with 2
RES_CASES = [("bf16-4096", 2, 97, 4096, 5, True), ("bf16-80", 3, 50, 80, 4, True),
             ("f32-64", 2, 64, 64, 3, False), ("bf16-8192", 1, 9, 8192, 2, True),
             ("bf16-3584", 2, 40, 3584, 4, True), ("f32-2048", 1, 33, 2048, 3, False),
             ("bf16-1040", 2, 21, 1040, 3, True), ("bf16-6160", 1, 7, 6160, 2, True),
             ("f32-4096", 1, 20, 4096, 3, False),
             ("bf16-2048-k200", 2, 300, 2048, 200, True)]   # many small clusters: a new centre almost every row


@pytest.mark.parametrize("grouped", [False, True], ids=["row-order", "grouped"])
@pytest.mark.parametrize("case", RES_CASES, ids=[c[0] for c in RES_CASES])
def test_residual_bit_exact(P, case, grouped):
    name, W, N, d, K, bf = case
    say("residual", name, "grouped" if grouped else "row order")
    rng = np.random.default_rng(11)
    H32 = (rng.standard_normal((W, N, d)) * np.exp(rng.uniform(-4, 4, (W, N, 1)))).astype(np.float32)
    H32[0, 1] = 0.0                                   # zero row
    H32[0, 2, 16:48] *= 1e-6                          # blocks far below the row max
    H32[0, 5] = 1e-40                                 # subnormal unit-row entries: the
    H32[0, 5, 0] = 1.0                                # coder's exact-division path
    H = O.f32_to_bf16(H32) if bf else H32
    Hf = bf16f(H) if bf else H
    rn = np.sqrt((Hf.astype(np.float64) ** 2).sum(-1)).astype(np.float32)
    C = rng.standard_normal((W, K, d)).astype(np.float32)
    C /= np.linalg.norm(C, axis=-1, keepdims=True)
    C[0, 1, 7] = np.nan                                 # non-finite residuals: exact path
    assign = rng.integers(0, K, (W, N)).astype(np.int32)
    assign[0, 3] = -5                                   # out of range reads cluster 0
    # a row whose residual is exactly zero: h = c * n with n = 1 exactly representable
    if not bf:
        C[0, 0] = 0
        C[0, 0, 0] = 1.0
        H[0, 4] = 0
        H[0, 4, 0] = 1.0
        rn[0, 4] = 1.0
        assign[0, 4] = 0
    s = P.Shape(W=W, N=N, d=d, K=K)
    dt = P.PS_BF16 if bf else P.PS_F32
    codes = torch.zeros(W, N, d // 2, dtype=torch.uint8, device="cuda")
    bsc = torch.zeros(W, N, d // 16, dtype=torch.uint8, device="cuda")
    rsc = torch.zeros(W, N, device="cuda")
    ws = torch.empty(8 * W * N + 16, dtype=torch.uint8, device="cuda") if grouped else None  # the minimum
    P.ps_residual_nvfp4(s, dt, dev(H), dev(rn), dev(C), dev(assign), codes, bsc, rsc, ws)
    torch.cuda.synchronize()
    r = O.residual_nvfp4(O.Shape(W=W, N=N, d=d, K=K), O.BF16 if bf else O.F32, H, rn, C, assign)
    assert np.array_equal(host(rsc).view(np.uint32), r["rscale"].view(np.uint32))
    assert np.array_equal(host(bsc), r["bscale"])
    assert np.array_equal(host(codes), r["codes"])


def test_residual_ties_and_saturation(P):
    """Rows built so that many elements land exactly on E2M1 midpoints and
    block scales on E4M3 midpoints and on the 448 saturation edge."""
    rng = np.random.default_rng(12)
    N, d = 256, 256
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.5, 3.0], np.float64)
    H = np.zeros((1, N, d), np.float32)
    for j in range(N):
        g = 2.0 ** rng.integers(-12, -2)
        for b in range(d // 16):
            sc = float(O.e4m3_decode(int(rng.integers(8, 126))))
            if rng.random() < 0.3:  # a scale exactly between two E4M3 values
                c0 = int(rng.integers(8, 125))
                sc = (float(O.e4m3_decode(c0)) + float(O.e4m3_decode(c0 + 1))) / 2
            v = rng.choice(mids, 16) * rng.choice([-1, 1], 16)
            v[0] = 6.0
            H[0, j, 16 * b:16 * b + 16] = (v * sc * g).astype(np.float32)
        H[0, j, 0] = np.float32(6.0 * 448 * g)
    rn = np.ones((1, N), np.float32)
    C = np.zeros((1, 1, d), np.float32)
    a = np.zeros((1, N), np.int32)
    s = P.Shape(W=1, N=N, d=d, K=1)
    codes = torch.zeros(1, N, d // 2, dtype=torch.uint8, device="cuda")
    bsc = torch.zeros(1, N, d // 16, dtype=torch.uint8, device="cuda")
    rsc = torch.zeros(1, N, device="cuda")
    P.ps_residual_nvfp4(s, P.PS_F32, dev(H), dev(rn), dev(C), dev(a), codes, bsc, rsc,
                        torch.empty(8 * N + 16, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    r = O.residual_nvfp4(O.Shape(W=1, N=N, d=d, K=1), O.F32, H, rn, C, a)
    assert np.array_equal(host(rsc).view(np.uint32), r["rscale"].view(np.uint32))
    assert np.array_equal(host(bsc), r["bscale"])
    assert np.array_equal(host(codes), r["codes"])


ATT_CASES = [
    # name, W, Nb, Hq, Hkv, dh, K, bf16
    ("llada", 2, 32, 32, 32, 128, 64, True),
    ("dream-gqa", 1, 32, 28, 4, 128, 128, True),
    ("ragged", 3, 13, 6, 3, 24, 37, True),
    ("k256", 1, 32, 8, 8, 128, 256, True),
    ("k128-nb5", 3, 5, 6, 3, 128, 128, True),      # one query block, 18 (window, head) pairs
    ("k256-nb50", 2, 50, 4, 2, 128, 256, True),    # four query blocks, the last ragged
    ("k200", 2, 20, 6, 2, 128, 200, True),         # head-split general kernel; ragged last score block
    ("k80-dh64", 1, 16, 4, 4, 64, 80, True),       # the same with dh = 64
    ("k32-nb20", 3, 20, 8, 2, 128, 32, True),      # a few windows below 65 clusters: head-parallel
    ("k16", 1, 8, 4, 4, 128, 16, True),
    ("k64-hq6-gqa", 2, 32, 6, 3, 128, 64, True),  # heads per wave stream uneven (2, 2, 1, 1)
    ("k256-mqa", 2, 32, 8, 1, 128, 256, True),     # one KV head for all query heads
    ("k256-nb64", 1, 64, 4, 4, 128, 256, True),    # the largest decode block the call accepts
    ("k64-nb64", 1, 64, 8, 8, 128, 64, True),
    ("k1000", 1, 5, 2, 1, 32, 1000, True),
    ("f32", 2, 16, 1, 1, 64, 8, False),
]


@pytest.mark.parametrize("case", ATT_CASES, ids=[c[0] for c in ATT_CASES])
@pytest.mark.parametrize("kind", [0, 1, 2])
def test_proxy_attn_and_drift(P, case, kind):
    name, W, Nb, Hq, Hkv, dh, K, bf = case
    say("proxy", name, kind)
    rng = np.random.default_rng(13)
    if bf:
        Q, Ck = rnd_bf16(rng, (W, Nb, Hq, dh)), rnd_bf16(rng, (W, K, Hkv, dh), 0.5)
    else:
        Q = rng.standard_normal((W, Nb, Hq, dh)).astype(np.float32)
        Ck = (rng.standard_normal((W, K, Hkv, dh)) * 0.5).astype(np.float32)
    s = P.Shape(W=W, N=K, d=16, Hq=Hq, Hkv=Hkv, dh=dh, Nb=Nb, K=K)
    so = O.Shape(W=W, N=K, d=16, Hq=Hq, Hkv=Hkv, dh=dh, Nb=Nb, K=K)
    sigma = float(np.float32(dh ** -0.5))
    prev = O.proxy_attn(so, O.BF16 if bf else O.F32, Q, Ck, sigma)["logp"]
    prev = (prev + rng.standard_normal(prev.shape).astype(np.float32) * 0.05).astype(np.float32)
    dt = P.PS_BF16 if bf else P.PS_F32
    lc = torch.zeros(W, Hq, Nb, K, device="cuda")
    Dhi = torch.zeros(W, Hq, Nb, device="cuda")
    Di = torch.zeros(W, Nb, device="cuda")
    sc = torch.zeros(W, K, device="cuda")
    P.ps_proxy_attn(s, dt, dev(Q), dev(Ck), sigma, lc, dev(prev), kind, Dhi, Di, sc)
    torch.cuda.synchronize()
    ro = O.proxy_attn(so, O.BF16 if bf else O.F32, Q, Ck, sigma)
    gl = host(lc)
    assert close(gl, ro["logp"]), f"logp {max_rel(gl, ro['logp'])}"
    kl = O.proxy_attn(so, O.BF16 if bf else O.F32, Q, Ck, sigma, prev, kind)
    assert close(host(Dhi), kl["D_hi"])
    assert close(host(Di), kl["D_i"])
    assert close(host(sc), kl["score"])
    # without D_hi (above 64 clusters the rows' drifts then cannot go through
    # it, and another kernel form runs): the same results
    Di2, sc2 = torch.zeros_like(Di), torch.zeros_like(sc)
    P.ps_proxy_attn(s, dt, dev(Q), dev(Ck), sigma, lc, dev(prev), kind, None, Di2, sc2)
    torch.cuda.synchronize()
    assert np.array_equal(host(lc), gl)
    assert close(host(Di2), kl["D_i"]) and close(host(sc2), kl["score"])
    if bf and K <= 64:
        # below 65 clusters both forms add the scores and D_i in one order
        assert np.array_equal(host(Di2).view(np.uint32), host(Di).view(np.uint32))
        assert np.array_equal(host(sc2).view(np.uint32), host(sc).view(np.uint32))
    # window formation: no previous distribution -> zeros, the same logits
    lc.zero_()
    P.ps_proxy_attn(s, dt, dev(Q), dev(Ck), sigma, lc, None, kind, Dhi, Di, sc)
    torch.cuda.synchronize()
    assert np.array_equal(host(lc), gl)
    assert not host(Di).any() and not host(sc).any() and not host(Dhi).any()


@pytest.mark.parametrize("Hkv", [32, 8])
def test_proxy_kernels_agree_bitwise(P, Hkv):
    """With two windows per compute unit and more, drift-step proxy attention
    at K = 64, dh = 128 runs the whole-row kernel (two waves per window); a
    single window runs the four-wave pipelined kernel.  Both add the same
    terms in the same order, so a window's log-probabilities, drifts and
    scores are bit-identical either way."""
    W = 2 * torch.cuda.get_device_properties(0).multi_processor_count
    Nb, Hq, dh, K = 32, 32, 128, 64
    say("proxy kernels agree", W, Hkv)
    g = torch.Generator(device="cuda").manual_seed(21)
    Q = torch.randn(W, Nb, Hq, dh, device="cuda", generator=g).to(torch.bfloat16)
    Ck = (torch.randn(W, K, Hkv, dh, device="cuda", generator=g) * 0.5).to(torch.bfloat16)
    prev = torch.log_softmax(torch.randn(W, Hq, Nb, K, device="cuda", generator=g) * 2.0, dim=-1)
    sigma = float(np.float32(dh ** -0.5))

    def run(sl, n):
        s = P.Shape(W=n, N=K, d=16, Hq=Hq, Hkv=Hkv, dh=dh, Nb=Nb, K=K)
        out = (torch.zeros(n, Hq, Nb, K, device="cuda"), torch.zeros(n, Hq, Nb, device="cuda"),
               torch.zeros(n, Nb, device="cuda"), torch.zeros(n, K, device="cuda"))
        P.ps_proxy_attn(s, P.PS_BF16, Q[sl].contiguous(), Ck[sl].contiguous(), sigma, out[0],
                        prev[sl].contiguous(), 0, out[1], out[2], out[3])
        torch.cuda.synchronize()
        return [host(x) for x in out]

    full = run(slice(0, W), W)
    for w in (0, 137 % W, W - 1):
        one = run(slice(w, w + 1), 1)
        for a, b in zip(full, one):
            assert np.array_equal(a[w].view(np.uint32), b[0].view(np.uint32)), f"window {w}"


def test_drift_identical_is_exactly_zero(P):
    rng = np.random.default_rng(14)
    W, Hq, Nb, K = 2, 8, 16, 64
    lp = O.proxy_attn(O.Shape(W=W, N=K, d=16, Hq=Hq, Hkv=Hq, dh=16, Nb=Nb, K=K), O.F32,
                      rng.standard_normal((W, Nb, Hq, 16)).astype(np.float32),
                      rng.standard_normal((W, K, Hq, 16)).astype(np.float32), 0.25)["logp"]
    s = P.Shape(W=W, N=K, d=16, Hq=Hq, Hkv=Hq, dh=16, Nb=Nb, K=K)
    Dhi, Di, sc = (torch.ones(W, Hq, Nb, device="cuda"), torch.ones(W, Nb, device="cuda"),
                   torch.ones(W, K, device="cuda"))
    P.ps_drift_kl(s, dev(lp), dev(lp.copy()), 0, Dhi, Di, sc)
    torch.cuda.synchronize()
    assert not host(Dhi).any() and not host(Di).any() and not host(sc).any()


@pytest.mark.parametrize("K,k", [(8, 2), (64, 4), (128, 8), (256, 16), (1000, 64), (5, 5), (1, 1)])
def test_topk_bit_exact(P, K, k):
    rng = np.random.default_rng(K * 7 + k)
    W = 9
    sc = rng.standard_normal((W, K)).astype(np.float32)
    sc[1, ::2] = 0.25                       # planted ties
    sc[2, : K // 2] = -0.0
    sc[2, K // 2:] = 0.0
    sc[3, rng.integers(0, K, max(1, K // 5))] = np.nan
    sc[4, 0] = np.inf
    sc[4, -1] = -np.inf
    sc[5, :] = np.nan
    sc[6] = np.round(sc[6], 1)              # many ties
    sc[7] = 1e-30 * sc[7]                   # subnormal-range scores
    s = P.Shape(W=W, N=K, d=16, K=K)
    idx = torch.zeros(W, k, dtype=torch.int32, device="cuda")
    val = torch.zeros(W, k, device="cuda")
    P.ps_topk_clusters(s, dev(sc), k, idx, val)
    torch.cuda.synchronize()
    r = O.topk_clusters(O.Shape(W=W, N=K, d=16, K=K), sc, k)
    assert np.array_equal(host(idx), r["idx"])
    assert np.array_equal(host(val), r["val"], equal_nan=True)


def pinned(a):
    """A new pinned host tensor (hipHostMalloc) holding a copy of a."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    out = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    out.copy_(t)
    return out


@pytest.mark.parametrize("bf,cap_mode,store", [(True, "ample", "device"), (True, "short", "device"),
                                               (True, "zero", "device"), (False, "ample", "device"),
                                               (False, "short", "device"), (False, "zero", "device"),
                                               (True, "ample", "host"), (False, "short", "host")])
def test_refresh_gather_bit_exact(P, bf, cap_mode, store):
    """Gather with the residual store in HBM or in pinned host memory (read
    across PCIe through its device mapping)."""
    rng = np.random.default_rng(15)
    W, N, d, K, k, Hkv, dh = 3, 517, 96, 23, 4, 2, 16
    H32 = rng.standard_normal((W, N, d)).astype(np.float32)
    H = O.f32_to_bf16(H32) if bf else H32
    Hf = bf16f(H) if bf else H
    rn = np.sqrt((Hf.astype(np.float64) ** 2).sum(-1)).astype(np.float32)
    C = rng.standard_normal((W, K, d)).astype(np.float32)
    C /= np.linalg.norm(C, axis=-1, keepdims=True)
    assign = rng.integers(0, K, (W, N)).astype(np.int32)
    so = O.Shape(W=W, N=N, d=d, Hq=Hkv, Hkv=Hkv, dh=dh, K=K)
    q = O.residual_nvfp4(so, O.BF16 if bf else O.F32, H, rn, C, assign)
    idx = np.stack([rng.choice(K, k, replace=False) for _ in range(W)]).astype(np.int32)
    idx[2, 0] = K + 3   # out of range: selects nothing
    idx[1, 1] = idx[1, 0]   # selected twice: selects it once
    Kc = rnd_bf16(rng, (W, N, Hkv, dh)) if bf else rng.standard_normal((W, N, Hkv, dh)).astype(np.float32)
    Vc = rnd_bf16(rng, (W, N, Hkv, dh)) if bf else rng.standard_normal((W, N, Hkv, dh)).astype(np.float32)
    cap = {"ample": N, "short": 17, "zero": 0}[cap_mode]
    r = O.refresh_gather(so, O.BF16 if bf else O.F32, assign, idx, k, cap, q["codes"], q["bscale"],
                         q["rscale"], C, rn, True, Kc, Vc)
    s = P.Shape(W=W, N=N, d=d, Hq=Hkv, Hkv=Hkv, dh=dh, K=K)
    et = torch.bfloat16 if bf else torch.float32
    pos = torch.full((W, max(cap, 1)), -1, dtype=torch.int32, device="cuda")
    count = torch.zeros(W, dtype=torch.int32, device="cuda")
    Hh = torch.zeros(W, max(cap, 1), d, dtype=et, device="cuda")
    Ko = torch.zeros(W, max(cap, 1), Hkv, dh, dtype=et, device="cuda")
    Vo = torch.zeros(W, max(cap, 1), Hkv, dh, dtype=et, device="cuda")
    put = pinned if store == "host" else dev
    P.ps_refresh_gather(s, P.PS_BF16 if bf else P.PS_F32, dev(assign), dev(idx), k, cap,
                        pos if cap else None, count, put(q["codes"]), put(q["bscale"]),
                        put(q["rscale"]), dev(C), dev(rn), Hh if cap else None,
                        dev(Kc) if cap else None, dev(Vc) if cap else None,
                        Ko if cap else None, Vo if cap else None)
    torch.cuda.synchronize()
    assert np.array_equal(host(count), r["count"])
    if cap:
        for w in range(W):
            m = min(int(r["count"][w]), cap)
            assert np.array_equal(host(pos)[w, :m], r["pos"][w, :m])
            assert np.array_equal(host(Hh)[w, :m].view(np.uint16 if bf else np.uint32),
                                  r["H_hat"][w, :m].view(np.uint16 if bf else np.uint32))
            assert np.array_equal(host(Ko)[w, :m], r["K_out"][w, :m])
            assert np.array_equal(host(Vo)[w, :m], r["V_out"][w, :m])
            assert np.all(host(pos)[w, m:] == -1)       # slots past count untouched


GATHER_PART_CASES = [
    # name, bf16, d, Hkv, dh, outputs (H_hat, K, V)
    ("d8192-all", True, 8192, 8, 128, (True, True, True)),      # two rounds of rebuilt chunks
    ("d8192-h-only", True, 8192, 8, 128, (True, False, False)),
    ("k-only", True, 4096, 32, 128, (False, True, False)),
    ("v-only", True, 4096, 32, 128, (False, False, True)),
    ("kv-long-rows", True, 256, 64, 160, (False, True, True)),   # 1280 pieces: three rounds
    ("f32-d4160-all", False, 4160, 4, 64, (True, True, True)),   # ragged second round
    ("d8320-h-only", True, 8320, 8, 128, (True, False, False)),  # centre past 8192 elements read per row
]


@pytest.mark.parametrize("case", GATHER_PART_CASES, ids=[c[0] for c in GATHER_PART_CASES])
def test_refresh_gather_rows_and_partial_outputs(P, case):
    """Rows longer than one round of the gather workgroup and every subset of
    the outputs (the kernel reads only what it writes)."""
    name, bf, d, Hkv, dh, (want_h, want_k, want_v) = case
    say("gather", name)
    rng = np.random.default_rng(d + Hkv)
    W, N, K, k = 2, 150, 6, 2
    H32 = rng.standard_normal((W, N, d)).astype(np.float32)
    H = O.f32_to_bf16(H32) if bf else H32
    Hf = bf16f(H) if bf else H
    rn = np.sqrt((Hf.astype(np.float64) ** 2).sum(-1)).astype(np.float32)
    C = rng.standard_normal((W, K, d)).astype(np.float32)
    C /= np.linalg.norm(C, axis=-1, keepdims=True)
    assign = rng.integers(0, K, (W, N)).astype(np.int32)
    so = O.Shape(W=W, N=N, d=d, Hq=Hkv, Hkv=Hkv, dh=dh, K=K)
    dt_o = O.BF16 if bf else O.F32
    q = O.residual_nvfp4(so, dt_o, H, rn, C, assign)
    idx = np.stack([rng.choice(K, k, replace=False) for _ in range(W)]).astype(np.int32)
    mk = (lambda: rnd_bf16(rng, (W, N, Hkv, dh))) if bf else \
        (lambda: rng.standard_normal((W, N, Hkv, dh)).astype(np.float32))
    Kc, Vc = mk(), mk()
    cap = N
    r = O.refresh_gather(so, dt_o, assign, idx, k, cap, q["codes"], q["bscale"], q["rscale"], C, rn,
                         want_h, Kc if want_k else None, Vc if want_v else None)
    s = P.Shape(W=W, N=N, d=d, Hq=Hkv, Hkv=Hkv, dh=dh, K=K)
    et = torch.bfloat16 if bf else torch.float32
    pos = torch.full((W, cap), -1, dtype=torch.int32, device="cuda")
    count = torch.zeros(W, dtype=torch.int32, device="cuda")
    Hh = torch.zeros(W, cap, d, dtype=et, device="cuda") if want_h else None
    Ko = torch.zeros(W, cap, Hkv, dh, dtype=et, device="cuda") if want_k else None
    Vo = torch.zeros(W, cap, Hkv, dh, dtype=et, device="cuda") if want_v else None
    P.ps_refresh_gather(s, P.PS_BF16 if bf else P.PS_F32, dev(assign), dev(idx), k, cap, pos, count,
                        dev(q["codes"]), dev(q["bscale"]), dev(q["rscale"]), dev(C), dev(rn), Hh,
                        dev(Kc) if want_k else None, dev(Vc) if want_v else None, Ko, Vo)
    torch.cuda.synchronize()
    assert np.array_equal(host(count), r["count"])
    u = np.uint16 if bf else np.uint32
    for w in range(W):
        m = int(r["count"][w])
        assert m > 0
        assert np.array_equal(host(pos)[w, :m], r["pos"][w, :m])
        if want_h:
            assert np.array_equal(host(Hh)[w, :m].view(u), r["H_hat"][w, :m].view(u))
            assert not host(Hh)[w, m:].any(), "rows past the count untouched"
        if want_k:
            assert np.array_equal(host(Ko)[w, :m].view(u), r["K_out"][w, :m].view(u))
            assert not host(Ko)[w, m:].any()
        if want_v:
            assert np.array_equal(host(Vo)[w, :m].view(u), r["V_out"][w, :m].view(u))
            assert not host(Vo)[w, m:].any()


def test_refresh_gather_many_windows(P):
    """Enough (window, selected cluster) pairs that each gets one workgroup
    (fewer pairs split a cluster's members over several)."""
    rng = np.random.default_rng(16)
    W, N, d, K, k, Hkv, dh = 160, 96, 64, 8, 4, 1, 16
    say("gather many windows", W)
    H = O.f32_to_bf16(rng.standard_normal((W, N, d)).astype(np.float32))
    rn = np.sqrt((bf16f(H).astype(np.float64) ** 2).sum(-1)).astype(np.float32)
    C = rng.standard_normal((W, K, d)).astype(np.float32)
    C /= np.linalg.norm(C, axis=-1, keepdims=True)
    assign = rng.integers(0, K, (W, N)).astype(np.int32)
    so = O.Shape(W=W, N=N, d=d, Hq=Hkv, Hkv=Hkv, dh=dh, K=K)
    q = O.residual_nvfp4(so, O.BF16, H, rn, C, assign)
    idx = np.stack([rng.choice(K, k, replace=False) for _ in range(W)]).astype(np.int32)
    Kc, Vc = rnd_bf16(rng, (W, N, Hkv, dh)), rnd_bf16(rng, (W, N, Hkv, dh))
    r = O.refresh_gather(so, O.BF16, assign, idx, k, N, q["codes"], q["bscale"], q["rscale"], C, rn, True, Kc, Vc)
    s = P.Shape(W=W, N=N, d=d, Hq=Hkv, Hkv=Hkv, dh=dh, K=K)
    pos = torch.full((W, N), -1, dtype=torch.int32, device="cuda")
    count = torch.zeros(W, dtype=torch.int32, device="cuda")
    Hh = torch.zeros(W, N, d, dtype=torch.bfloat16, device="cuda")
    Ko = torch.zeros(W, N, Hkv, dh, dtype=torch.bfloat16, device="cuda")
    Vo = torch.zeros(W, N, Hkv, dh, dtype=torch.bfloat16, device="cuda")
    P.ps_refresh_gather(s, P.PS_BF16, dev(assign), dev(idx), k, N, pos, count, dev(q["codes"]),
                        dev(q["bscale"]), dev(q["rscale"]), dev(C), dev(rn), Hh, dev(Kc), dev(Vc), Ko, Vo)
    torch.cuda.synchronize()
    assert np.array_equal(host(count), r["count"])
    for w in range(W):
        m = int(r["count"][w])
        assert np.array_equal(host(pos)[w, :m], r["pos"][w, :m])
        assert np.array_equal(host(Hh)[w, :m].view(np.uint16), r["H_hat"][w, :m].view(np.uint16))
        assert np.array_equal(host(Ko)[w, :m], r["K_out"][w, :m])
        assert np.array_equal(host(Vo)[w, :m], r["V_out"][w, :m])


def test_w_zero_is_a_no_op(P):
    s = P.Shape(W=0, N=64, d=32, K=4)
    z = torch.zeros(16, dtype=torch.int32, device="cuda")
    P.ps_topk_clusters(s, torch.zeros(16, device="cuda"), 2, z)
    torch.cuda.synchronize()


def cosine_close(got, want, d):
    """fp32 roundings of 1 - (a fp64 dot product of unit vectors summed in two
    different orders): the fp64 sums differ by at most d * 2^-53 * sum|a b|
    <= d * 2^-53, and each side rounds once to fp32 (one fp32 ulp)."""
    got, want = np.asarray(got, np.float32), np.asarray(want, np.float32)
    tol = np.spacing(np.abs(want)).astype(np.float64) + d * 2.0 ** -53
    return bool(np.all(np.abs(got.astype(np.float64) - want) <= tol))


@pytest.mark.parametrize("W,K,d", [(3, 37, 80), (2, 64, 4096), (1, 1000, 16), (4, 1, 3584)])
def test_drift_cosine(P, W, K, d):
    rng = np.random.default_rng(W * 1000 + K)
    prev = rng.standard_normal((W, K, d))
    prev /= np.linalg.norm(prev, axis=-1, keepdims=True)
    cur = prev + rng.uniform(0, 0.3, (W, K, 1)) * rng.standard_normal((W, K, d)) / np.sqrt(d)
    cur /= np.linalg.norm(cur, axis=-1, keepdims=True)
    cur, prev = cur.astype(np.float32), prev.astype(np.float32)
    cur[0, 0] = prev[0, 0]                         # unmoved: exactly zero
    if K > 2:
        cur[0, 1] = -prev[0, 1]                    # reversed
    s = P.Shape(W=W, N=K, d=d, K=K)
    sc = torch.full((W, K), 7.0, device="cuda")
    P.ps_drift_cosine(s, dev(cur), dev(prev), sc)
    torch.cuda.synchronize()
    want = O.drift_cosine(O.Shape(W=W, N=K, d=d, K=K), cur, prev)
    got = host(sc)
    assert cosine_close(got, want, d), f"max diff {np.abs(got - want).max()}"
    # the unmoved centre scores 1 - ||c||^2: zero up to its fp32 normalisation
    assert abs(got[0, 0]) < 1e-6


def test_maximum_window_length(P):
    """The longest window the calls accept (N = 2^24 - 1 rows, ragged against
    every tile size), with planted, well-separated clusters so that no row is
    a near-tie: K-Means from farthest-first seeds, then the NVFP4 coder, the
    gather of one cluster and the suffix commit rule on the oracle's own
    clustering, each against the oracle."""
    N, d, K = (1 << 24) - 1, 16, 3
    rng = np.random.default_rng(24)
    u = rng.standard_normal((K, d))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    x = (u[rng.integers(0, K, N)] + 0.05 * rng.standard_normal((N, d))).astype(np.float32)
    xb = x.view(np.uint32)
    H = ((xb + 0x7FFF + ((xb >> 16) & 1)) >> 16).astype(np.uint16).reshape(1, N, d)
    del x, xb
    Kr = H.reshape(1, N, 1, d)
    s = P.Shape(W=1, N=N, d=d, Hq=1, Hkv=1, dh=d, Nb=32, K=K)
    so = O.Shape(W=1, N=N, d=d, Hq=1, Hkv=1, dh=d, Nb=32, K=K)
    say("maximum window: oracle K-Means")
    r = O.kmeans_fit(so, O.BF16, H, Kr, O.INIT_FARTHEST, 2, np.zeros((1, K, d), np.float32))
    Hd, Krd = dev(H), dev(Kr)
    C = torch.zeros(1, K, d, device="cuda")
    a = torch.zeros(1, N, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(1, K, dtype=torch.int32, device="cuda")
    rn = torch.zeros(1, N, device="cuda")
    Ck = torch.zeros(1, K, 1, d, dtype=torch.bfloat16, device="cuda")
    obj = torch.zeros(1, dtype=torch.float64, device="cuda")
    ws = P.workspace(s, P.PS_BF16)
    P.ps_kmeans_fit(s, P.PS_BF16, Hd, Krd, P.PS_INIT_FARTHEST, 2, C, a, cnt, rn, Ck, obj, ws)
    torch.cuda.synchronize()
    assert max_rel(host(rn), r["row_norm"]) <= 1.2e-7, "row norms"
    assert np.array_equal(host(a), r["assign"]), "assignments"
    assert np.array_equal(host(cnt), r["counts"]), "counts"
    assert close(host(C), r["C"], 1e-6, 1e-7), "centres"
    assert np.array_equal(host(Ck), r["Ck"]), "centroid keys"

    say("maximum window: NVFP4 coder")
    q = O.residual_nvfp4(so, O.BF16, H, r["row_norm"], r["C"], r["assign"])
    codes = torch.zeros(1, N, d // 2, dtype=torch.uint8, device="cuda")
    bscale = torch.zeros(1, N, d // 16, dtype=torch.uint8, device="cuda")
    rscale = torch.zeros(1, N, device="cuda")
    rn_o, C_o, a_o = dev(r["row_norm"]), dev(r["C"]), dev(r["assign"])
    P.ps_residual_nvfp4(s, P.PS_BF16, Hd, rn_o, C_o, a_o, codes, bscale, rscale, ws=ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(codes), q["codes"]), "codes"
    assert np.array_equal(host(bscale), q["bscale"]), "block scales"
    assert np.array_equal(host(rscale).view(np.uint32), q["rscale"].view(np.uint32)), "row scales"
    del codes, bscale, rscale

    say("maximum window: gather of one cluster")
    idx = np.array([[1]], np.int32)
    cap = 6_000_000                                   # above the ~N/3 members of a cluster
    g = O.refresh_gather(so, O.BF16, r["assign"], idx, 1, cap, q["codes"], q["bscale"], q["rscale"], r["C"],
                         r["row_norm"], True, Kr, None)
    pos = torch.full((1, cap), -1, dtype=torch.int32, device="cuda")
    count = torch.zeros(1, dtype=torch.int32, device="cuda")
    Hh = torch.zeros(1, cap, d, dtype=torch.bfloat16, device="cuda")
    Ko = torch.zeros(1, cap, 1, d, dtype=torch.bfloat16, device="cuda")
    P.ps_refresh_gather(s, P.PS_BF16, a_o, dev(idx), 1, cap, pos, count, dev(q["codes"]), dev(q["bscale"]),
                        dev(q["rscale"]), C_o, rn_o, Hh, Krd, None, Ko, None)
    torch.cuda.synchronize()
    m = int(g["count"][0])
    assert 0 < m <= cap and int(host(count)[0]) == m
    assert np.array_equal(host(pos)[0, :m], g["pos"][0, :m])
    assert np.array_equal(host(Hh)[0, :m], g["H_hat"][0, :m])
    assert np.array_equal(host(Ko)[0, :m], g["K_out"][0, :m])
    del pos, Hh, Ko

    say("maximum window: suffix commit rule")
    b0 = N // 2 - 16
    conf = rng.random((1, N), dtype=np.float32)
    cs = O.commit_suffix(so, r["assign"], idx, 1, b0, conf, 0.9)
    flag = torch.zeros(1, dtype=torch.uint8, device="cuda")
    commit = torch.zeros(1, N, dtype=torch.uint8, device="cuda")
    P.ps_commit_suffix(s, a_o, dev(idx), 1, b0, dev(conf), 0.9, flag, commit)
    torch.cuda.synchronize()
    assert np.array_equal(host(flag), cs["flag"]) and np.array_equal(host(commit), cs["commit"])
