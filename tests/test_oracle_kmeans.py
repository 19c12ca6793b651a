"""Pins of the oracle's spherical K-Means (init, Lloyd iterations, centroid
keys) against planted structure, closed forms, invariants and brute force."""
import itertools

import numpy as np
import pytest

import oracle as O
import synth


def _unit(H):
    H = H.astype(np.float64)
    n = np.sqrt((H * H).sum(-1, keepdims=True))
    return H / np.where(n > 0, n, 1)


def _bf16_to_f32(b):
    return (b.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_planted_recovery_farthest(seed):
    cfg = synth.CONFIGS["tiny-planted"]
    data = synth.generate(cfg, seed=synth.BASE_SEED + 1000 * seed)
    s = O.Shape(W=1, N=cfg.N, d=cfg.d, Hq=1, Hkv=1, dh=cfg.dh, Nb=cfg.Nb, K=cfg.K)
    C = np.zeros((1, cfg.K, cfg.d), np.float32)
    r = O.kmeans_fit(s, O.F32, data["H"], data["Kr"], O.INIT_FARTHEST, cfg.iters, C)
    lab, a = data["labels"][0], r["assign"][0]
    # same partition up to a permutation of cluster ids
    m = {}
    for x, y in zip(lab.tolist(), a.tolist()):
        assert m.setdefault(x, y) == y
    assert len(set(m.values())) == cfg.K


def test_farthest_seeds_hit_every_planted_direction():
    cfg = synth.CONFIGS["tiny-planted"]
    data = synth.generate(cfg)
    s = O.Shape(W=1, N=cfg.N, d=cfg.d, K=cfg.K)
    C = O.kmeans_init(s, O.F32, data["H"], O.INIT_FARTHEST)[0]
    X = _unit(data["H"][0])
    sim = X @ C.astype(np.float64).T
    seeds = sim.argmax(0).tolist()
    assert np.all(sim.max(0) > 1 - 1e-6)    # every centre is one of the unit rows
    assert seeds[0] == 0
    assert sorted(data["labels"][0][seeds].tolist()) == list(range(cfg.K))


def test_strided_init_rows():
    rng = np.random.default_rng(5)
    N, d, K = 37, 32, 5
    H = rng.standard_normal((1, N, d)).astype(np.float32)
    C = O.kmeans_init(O.Shape(W=1, N=N, d=d, K=K), O.F32, H, O.INIT_STRIDED)[0]
    n = np.sqrt((H[0].astype(np.float64) ** 2).sum(-1)).astype(np.float32)
    for k in range(K):
        j = (k * N) // K
        assert np.array_equal(C[k], (H[0, j] / n[j]).astype(np.float32))


def test_objective_non_decreasing_fp32():
    """Dhillon-Modha: each assignment and each update can only raise
    sum_k ||S_k|| (fp32 path, where the assignment uses the exact centres)."""
    rng = np.random.default_rng(6)
    N, d, K = 300, 48, 7
    H = rng.standard_normal((1, N, d)).astype(np.float32)
    s = O.Shape(W=1, N=N, d=d, K=K)
    C = O.kmeans_init(s, O.F32, H, O.INIT_STRIDED)
    objs, changes, prev = [], [], None
    for _ in range(15):
        r = O.kmeans_fit(s, O.F32, H, None, O.INIT_GIVEN, 1, C)
        objs.append(r["objective"][0])
        if prev is not None:
            changes.append(int((prev != r["assign"]).sum()))
        prev = r["assign"].copy()
    assert all(b >= a - 1e-9 * abs(a) for a, b in zip(objs, objs[1:])), objs
    assert objs[-1] > objs[0]
    assert changes[-1] == 0  # converged


def test_iterations_compose():
    """fit(iters=n) == fit(iters=1) applied n times (the only Lloyd state is C)."""
    rng = np.random.default_rng(7)
    N, d, K = 200, 64, 6
    H = O.f32_to_bf16(rng.standard_normal((1, N, d)).astype(np.float32))
    s = O.Shape(W=1, N=N, d=d, K=K)
    C0 = O.kmeans_init(s, O.BF16, H, O.INIT_STRIDED)
    A = O.kmeans_fit(s, O.BF16, H, None, O.INIT_GIVEN, 4, C0.copy())
    C = C0.copy()
    for _ in range(4):
        B = O.kmeans_fit(s, O.BF16, H, None, O.INIT_GIVEN, 1, C)
    assert np.array_equal(A["C"], B["C"])
    assert np.array_equal(A["assign"], B["assign"])


def test_k1_is_normalised_mean():
    rng = np.random.default_rng(8)
    N, d = 50, 32
    H = rng.standard_normal((1, N, d)).astype(np.float32)
    s = O.Shape(W=1, N=N, d=d, K=1)
    r = O.kmeans_fit(s, O.F32, H, None, O.INIT_STRIDED, 2, np.zeros((1, 1, d), np.float32))
    m = _unit(H[0]).sum(0)
    m /= np.linalg.norm(m)
    assert np.allclose(r["C"][0, 0], m, rtol=0, atol=2e-7)
    assert np.all(r["assign"] == 0) and r["counts"][0, 0] == N


def test_centres_are_unit_and_member_means():
    """Returned C is consistent with returned assign: every non-empty c_k is the
    normalised mean of its members' unit rows; ||c_k|| = 1."""
    rng = np.random.default_rng(9)
    N, d, K = 400, 64, 9
    H = O.f32_to_bf16(rng.standard_normal((1, N, d)).astype(np.float32))
    s = O.Shape(W=1, N=N, d=d, K=K)
    r = O.kmeans_fit(s, O.BF16, H, None, O.INIT_STRIDED, 3, np.zeros((1, K, d), np.float32))
    X = _unit(_bf16_to_f32(H[0]))
    a = r["assign"][0]
    assert r["counts"][0].sum() == N
    for k in range(K):
        mem = X[a == k]
        assert mem.shape[0] == r["counts"][0, k]
        if mem.shape[0]:
            m = mem.sum(0)
            m /= np.linalg.norm(m)
            assert np.allclose(r["C"][0, k], m, atol=1e-7)
    assert np.allclose(np.linalg.norm(r["C"][0].astype(np.float64), axis=1), 1, atol=1e-6)


def test_converged_assignment_is_argmax():
    """At a fixed point every row sits with its most similar (bf16-rounded)
    centre, checked by brute force over all K."""
    rng = np.random.default_rng(10)
    N, d, K = 256, 32, 5
    H = O.f32_to_bf16(rng.standard_normal((1, N, d)).astype(np.float32))
    s = O.Shape(W=1, N=N, d=d, K=K)
    C = O.kmeans_init(s, O.BF16, H, O.INIT_STRIDED)
    prev = None
    for _ in range(40):
        r = O.kmeans_fit(s, O.BF16, H, None, O.INIT_GIVEN, 1, C)
        if prev is not None and np.array_equal(prev, r["assign"]):
            break
        prev = r["assign"].copy()
    # one more iteration from the fixed point: nothing moves
    Cc = C.copy()
    r2 = O.kmeans_fit(s, O.BF16, H, None, O.INIT_GIVEN, 1, Cc)
    assert np.array_equal(r2["assign"], r["assign"]) and np.array_equal(Cc, C)
    Hf = _bf16_to_f32(H[0]).astype(np.float64)
    Cb = _bf16_to_f32(O.f32_to_bf16(C[0])).astype(np.float64)
    sc = Hf @ Cb.T
    assert np.array_equal(r["assign"][0], sc.argmax(1))


def test_brute_force_partition_optimum_tiny():
    """N = 8, K = 2, two well-separated groups: Lloyd from farthest-first
    reaches the best of all 2^N partitions; on random tiny data it never beats
    it."""
    rng = np.random.default_rng(11)
    d = 16
    base = rng.standard_normal((2, d))
    H = np.concatenate([base[0] + 0.1 * rng.standard_normal((4, d)),
                        base[1] + 0.1 * rng.standard_normal((4, d))]).astype(np.float32)
    for Hm, must_equal in ((H, True), (rng.standard_normal((8, d)).astype(np.float32), False)):
        X = _unit(Hm)
        best = -1.0
        for bits in itertools.product([0, 1], repeat=8):
            b = np.array(bits)
            v = sum(np.linalg.norm(X[b == k].sum(0)) for k in (0, 1) if (b == k).any())
            best = max(best, v)
        s = O.Shape(W=1, N=8, d=d, K=2)
        r = O.kmeans_fit(s, O.F32, Hm[None], None, O.INIT_FARTHEST, 20,
                         np.zeros((1, 2, d), np.float32))
        # the oracle divides by the fp32-rounded norm: relative slack 1e-6
        assert r["objective"][0] <= best * (1 + 1e-6)
        if must_equal:
            assert abs(r["objective"][0] - best) < 1e-6 * best


def test_empty_cluster_keeps_centre_and_key():
    rng = np.random.default_rng(12)
    N, d, K = 64, 32, 3
    H = np.abs(rng.standard_normal((1, N, d))).astype(np.float32)  # all in one orthant
    Kr = rng.standard_normal((1, N, 2, 16)).astype(np.float32)
    C = np.zeros((1, K, d), np.float32)
    C[0, 0] = _unit(H[0, :1])[0]
    C[0, 1] = -C[0, 0]                      # nobody is closest to the antipode
    C[0, 2] = _unit(H[0, 1:2])[0]
    Ck = np.full((1, K, 2, 16), 7.0, np.float32)
    s = O.Shape(W=1, N=N, d=d, Hq=2, Hkv=2, dh=16, K=K)
    anti = C[0, 1].copy()
    r = O.kmeans_fit(s, O.F32, H, Kr, O.INIT_GIVEN, 2, C, Ck)
    assert r["counts"][0, 1] == 0
    assert np.array_equal(r["C"][0, 1], anti)
    assert np.all(r["Ck"][0, 1] == 7.0)


def test_centroid_keys_are_member_means_bf16():
    rng = np.random.default_rng(13)
    N, d, K, Hkv, dh = 128, 32, 4, 2, 16
    H = O.f32_to_bf16(rng.standard_normal((1, N, d)).astype(np.float32))
    Kr = O.f32_to_bf16(rng.standard_normal((1, N, Hkv, dh)).astype(np.float32))
    s = O.Shape(W=1, N=N, d=d, Hq=4, Hkv=Hkv, dh=dh, K=K)
    r = O.kmeans_fit(s, O.BF16, H, Kr, O.INIT_STRIDED, 3, np.zeros((1, K, d), np.float32))
    Krf = _bf16_to_f32(Kr[0]).astype(np.float64)
    Ckf = _bf16_to_f32(r["Ck"][0]).astype(np.float64)
    a = r["assign"][0]
    for k in range(K):
        mean = Krf[a == k].mean(0)
        # one bf16 rounding: relative error <= 2^-8
        assert np.all(np.abs(Ckf[k] - mean) <= 2.0 ** -8 * np.abs(mean) + 1e-30)


def test_k_equals_n_gives_rows_and_exact_keys():
    """K = N with strided seeding (floor(kN/N) = k) on distinct random rows:
    every row is its own cluster, centres equal the unit rows (to rounding)
    and the centroid keys equal the key rows exactly."""
    rng = np.random.default_rng(14)
    N, d, Hkv, dh = 24, 64, 2, 8
    H = O.f32_to_bf16(rng.standard_normal((1, N, d)).astype(np.float32))
    Kr = O.f32_to_bf16(rng.standard_normal((1, N, Hkv, dh)).astype(np.float32))
    s = O.Shape(W=1, N=N, d=d, Hq=2, Hkv=Hkv, dh=dh, K=N)
    r = O.kmeans_fit(s, O.BF16, H, Kr, O.INIT_STRIDED, 1, np.zeros((1, N, d), np.float32))
    assert np.array_equal(r["assign"][0], np.arange(N))
    assert np.array_equal(r["Ck"], Kr)
    assert np.allclose(r["C"][0], _unit(_bf16_to_f32(H[0])), atol=1e-7)


def test_zero_row_is_harmless():
    rng = np.random.default_rng(15)
    N, d, K = 40, 32, 4
    H = rng.standard_normal((1, N, d)).astype(np.float32)
    H[0, 3] = 0.0
    s = O.Shape(W=1, N=N, d=d, K=K)
    r = O.kmeans_fit(s, O.F32, H, None, O.INIT_FARTHEST, 3, np.zeros((1, K, d), np.float32))
    assert np.isfinite(r["C"]).all() and r["row_norm"][0, 3] == 0.0
    assert r["assign"][0, 3] == 0  # all scores zero: lowest index


def test_row_norms_fp64_exact_on_small_integers():
    H = np.array([[[3.0, 4.0] + [0.0] * 14, [1.0] * 16]], np.float32)
    rn = O.row_norms(O.Shape(W=1, N=2, d=16), O.F32, H)
    assert rn[0, 0] == 5.0 and rn[0, 1] == 4.0


def test_argument_errors():
    s = O.Shape(W=1, N=8, d=16, K=9)
    H = np.zeros((1, 8, 16), np.float32)
    with pytest.raises(O.OracleError):
        O.kmeans_fit(s, O.F32, H, None, O.INIT_STRIDED, 1, np.zeros((1, 9, 16), np.float32))
    s = O.Shape(W=1, N=8, d=24, K=2)
    with pytest.raises(O.OracleError):
        O.kmeans_fit(s, O.F32, np.zeros((1, 8, 24), np.float32), None, O.INIT_STRIDED, 1,
                     np.zeros((1, 2, 24), np.float32))
    s = O.Shape(W=1, N=8, d=16, K=2)
    with pytest.raises(O.OracleError):
        O.kmeans_fit(s, O.F32, H, None, O.INIT_STRIDED, 0, np.zeros((1, 2, 16), np.float32))


def test_update_step_alone_matches_fit_and_member_means():
    """pso_kmeans_update from an assignment gives the normalised member means,
    and one fit iteration equals update(assign of that iteration)."""
    rng = np.random.default_rng(16)
    N, d, K = 300, 48, 6
    H = O.f32_to_bf16(rng.standard_normal((1, N, d)).astype(np.float32))
    s = O.Shape(W=1, N=N, d=d, K=K)
    C0 = O.kmeans_init(s, O.BF16, H, O.INIT_STRIDED)
    r = O.kmeans_fit(s, O.BF16, H, None, O.INIT_GIVEN, 1, C0.copy())
    u = O.kmeans_update(s, O.BF16, H, r["row_norm"], r["assign"], C0)
    assert np.array_equal(u["C"], r["C"]) and np.array_equal(u["counts"], r["counts"])
    assert u["objective"][0] == r["objective"][0]
    # arbitrary assignment with an empty cluster
    a = rng.integers(0, K - 1, size=(1, N)).astype(np.int32)
    u = O.kmeans_update(s, O.BF16, H, r["row_norm"], a, C0)
    X = _unit(_bf16_to_f32(H[0]))
    for k in range(K - 1):
        m = X[a[0] == k].sum(0)
        assert np.allclose(u["C"][0, k], m / np.linalg.norm(m), atol=1e-7)
    assert np.array_equal(u["C"][0, K - 1], C0[0, K - 1]) and u["counts"][0, K - 1] == 0
    with pytest.raises(O.OracleError):
        O.kmeans_update(s, O.BF16, H, r["row_norm"], np.full((1, N), K, np.int32), C0)


def test_assignment_ties_go_to_lowest_index():
    """Exactly equal scores (a duplicated centre, a row equidistant from two
    centres) go to the lowest cluster index."""
    d = 16
    e = np.eye(d, dtype=np.float32)
    H = np.stack([e[1], e[1] + e[0], e[2], e[0]])[None].astype(np.float32)      # [1][4][16]
    C = np.stack([e[0], e[1], e[1], e[2]])[None].astype(np.float32)             # centres 1 and 2 identical
    s = O.Shape(W=1, N=4, d=d, K=4)
    r = O.kmeans_fit(s, O.F32, H, None, O.INIT_GIVEN, 1, C.copy())
    # row 0 = e1: ties between centres 1 and 2 -> 1; row 1 = e0 + e1: ties
    # between 0 (score 1) and 1, 2 (score 1) -> 0; row 2 = e2 -> 3; row 3 = e0 -> 0
    assert r["assign"][0].tolist() == [1, 0, 3, 0]


def test_assignment_uses_bf16_rounded_centres():
    """On the bf16 path the scores use the centres rounded to bf16: two centres
    whose first components 1.00389 and 1.0039 both round to 1.0 tie, so the
    lower index wins, although the unrounded second centre scores higher."""
    d = 16
    H32 = np.zeros((1, 2, d), np.float32)
    H32[0, :, 0] = 1.0
    H = O.f32_to_bf16(H32)
    C = np.zeros((1, 2, d), np.float32)
    C[0, 0, 0] = np.float32(1.00389)
    C[0, 1, 0] = np.float32(1.0039)
    assert O.bf16_to_f32(O.f32_to_bf16(C[0, :, 0])).tolist() == [1.0, 1.0]
    s = O.Shape(W=1, N=2, d=d, K=2)
    r = O.kmeans_fit(s, O.BF16, H, None, O.INIT_GIVEN, 1, C.copy())
    assert r["assign"][0].tolist() == [0, 0]
    rf = O.kmeans_fit(s, O.F32, H32, None, O.INIT_GIVEN, 1, C.copy())
    assert rf["assign"][0].tolist() == [1, 1]            # fp32 path: no rounding, the larger wins


def test_singleton_cluster_centre_is_its_row():
    """A cluster with one member moves to that member's unit row, whatever
    centre it started from."""
    d = 16
    e = np.eye(d, dtype=np.float32)
    H = np.stack([e[0] + 0.25 * e[2], e[1] - 0.5 * e[3]])[None].astype(np.float32)
    C = np.stack([e[0], e[1]])[None].astype(np.float32)
    s = O.Shape(W=1, N=2, d=d, K=2)
    r = O.kmeans_fit(s, O.F32, H, None, O.INIT_GIVEN, 1, C.copy())
    assert r["assign"][0].tolist() == [0, 1]
    want = _unit(H[0]).astype(np.float32)
    assert np.allclose(r["C"][0], want, rtol=0, atol=1e-7)
    assert r["counts"][0].tolist() == [1, 1]
