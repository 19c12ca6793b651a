"""Pins of the oracle's cosine-dissimilarity drift (technical summary 2.A,
drift measurement: the cosine measure the KL drift is compared against), read
as 1 - <c_k(t), c_k(t-1)> of a cluster's unit centres between steps."""
import numpy as np
import pytest
from scipy.spatial import distance

import oracle as O


def _unit(rng, shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def test_identical_opposite_orthogonal_are_exact():
    d, K = 64, 3
    s = O.Shape(W=1, N=K, d=d, K=K)
    E = np.eye(d, dtype=np.float32)
    cur = np.stack([E[0], E[1], E[2]])[None]
    prev = np.stack([E[0], -E[1], E[5]])[None]
    sc = O.drift_cosine(s, np.ascontiguousarray(cur), np.ascontiguousarray(prev))
    assert sc[0].tolist() == [0.0, 2.0, 1.0]


def test_rotation_by_theta_gives_one_minus_cos_theta():
    rng = np.random.default_rng(2)
    W, K, d = 3, 5, 256
    thetas = rng.uniform(0, np.pi, size=(W, K))
    prev = _unit(rng, (W, K, d))
    g = rng.standard_normal((W, K, d))
    u = g - (g * prev).sum(-1, keepdims=True) * prev
    u /= np.linalg.norm(u, axis=-1, keepdims=True)
    cur = np.cos(thetas)[..., None] * prev + np.sin(thetas)[..., None] * u
    s = O.Shape(W=W, N=K, d=d, K=K)
    sc = O.drift_cosine(s, cur.astype(np.float32), prev.astype(np.float32))
    assert np.allclose(sc, 1.0 - np.cos(thetas), atol=2e-6)


def test_matches_scipy_cosine_distance_per_window_and_cluster():
    rng = np.random.default_rng(3)
    W, K, d = 2, 7, 96
    cur = _unit(rng, (W, K, d)).astype(np.float32)
    prev = _unit(rng, (W, K, d)).astype(np.float32)
    # nearly unmoved centres too: the small-angle end where cancellation bites
    near = cur[1, :3] + 1e-4 * rng.standard_normal((3, d))
    prev[1, :3] = (near / np.linalg.norm(near, axis=-1, keepdims=True)).astype(np.float32)
    s = O.Shape(W=W, N=K, d=d, K=K)
    sc = O.drift_cosine(s, cur, prev)
    for w in range(W):
        for k in range(K):
            a, b = cur[w, k].astype(np.float64), prev[w, k].astype(np.float64)
            # scipy normalises; the centres are unit vectors up to fp32 rounding
            want = distance.cosine(a, b)
            assert sc[w, k] == pytest.approx(want, rel=1e-5, abs=1e-6)


def test_rejects_bad_arguments():
    with pytest.raises(O.OracleError):
        O.drift_cosine(O.Shape(W=1, N=1, d=16, K=0), np.zeros((1, 1, 16), np.float32),
                       np.zeros((1, 1, 16), np.float32))
