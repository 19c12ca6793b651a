"""Pins of the oracle's Polestar-Commit rules (technical summary section 2.B,
current-block and suffix-block commitment items).

The current-block rule: a block row commits when its drift delta (drift now
minus the mean of its earlier drifts) exceeds alpha * (tau_s - c)^2, or when
its confidence c reaches tau_s.  The suffix rule: when a top-k drifted cluster
is a suffix-window cluster, suffix rows with c >= tau_s commit.

The worked cases below were derived by hand from those statements, with
values that are exact in binary where a comparison sits on its boundary.
"""
import numpy as np
import pytest

import oracle as O


def _block(D_rows, conf_rows, alpha, tau_s, hist_sum=None, hist_n=None):
    """One window, len(D_rows) block rows starting at position 0."""
    Nb = len(D_rows)
    s = O.Shape(W=1, N=max(Nb, 1), d=16, Nb=Nb, K=1)
    hs = np.zeros((1, Nb)) if hist_sum is None else hist_sum
    hn = np.zeros(1, np.int32) if hist_n is None else hist_n
    r = O.commit_block(s, np.array([D_rows], np.float32), np.array([conf_rows], np.float32), 0,
                       alpha, tau_s, hs, hn)
    return r, hs, hn


def _run_history(Ds, c, alpha, tau_s):
    """Feed a drift sequence to one row with fixed confidence; return the
    commit codes and deltas of every step."""
    hs, hn = np.zeros((1, 1)), np.zeros(1, np.int32)
    out = []
    for D in Ds:
        r, hs, hn = _block([D], [c], alpha, tau_s, hs, hn)
        out.append((int(r["commit"][0, 0]), float(r["delta"][0, 0])))
    return out, hs, hn


# ---- current block: hand-worked cases ----------------------------------------
def test_worked_case_delta_against_earlier_mean():
    # history 0.1, 0.3 -> mean 0.2; now 0.37 -> delta 0.17 > 1 * (0.9 - 0.5)^2 = 0.16
    out, _, _ = _run_history([0.1, 0.3, 0.37], 0.5, 1.0, 0.9)
    assert [o[0] for o in out] == [0, 1, 1]
    assert out[2][1] == pytest.approx(0.17, abs=1e-6)
    # now 0.35 -> delta 0.15 < 0.16: no commit.  (A mean that included the
    # current step, (0.1+0.3+0.37)/3, or an unsquared gap 0.4, or the gap
    # taken as c instead of tau_s - c, would all flip the 0.37 case.)
    out, _, _ = _run_history([0.1, 0.3, 0.35], 0.5, 1.0, 0.9)
    assert [o[0] for o in out] == [0, 1, 0]


def test_first_step_has_no_history():
    out, hs, hn = _run_history([5.0], 0.0, 0.0, 0.9)
    assert out == [(0, 0.0)]
    assert hn[0] == 1 and hs[0, 0] == 5.0


def test_threshold_is_strict_and_confidence_is_inclusive():
    # exact binary values: alpha=1, tau_s=0.75, c=0.25 -> threshold 0.25;
    # history 0.5, now 0.75 -> delta exactly 0.25: not above the threshold
    out, _, _ = _run_history([0.5, 0.75], 0.25, 1.0, 0.75)
    assert out[1] == (0, 0.25)
    above = float(np.nextafter(np.float32(0.75), np.float32(1.0)))
    out, _, _ = _run_history([0.5, above], 0.25, 1.0, 0.75)
    assert out[1][0] == 1
    # c == tau_s commits by the confidence rule (bit 1) even with no history
    r, _, _ = _block([0.0], [0.75], 1.0, 0.75)
    assert r["commit"][0, 0] == 2


def test_negative_delta_never_fires_with_zero_alpha():
    # alpha = 0: the drift rule is delta > 0
    out, _, _ = _run_history([1.0, 2.0, 1.0, 1.5, 1.33333337], 0.1, 0.0, 0.9)
    # means before each step: -, 1, 1.5, 4/3, 1.375
    assert [o[0] for o in out] == [0, 1, 0, 1, 0]


def test_two_bits_are_independent():
    # c >= tau_s and a large positive delta: both bits
    out, _, _ = _run_history([0.0, 10.0], 0.95, 1.0, 0.9)
    assert out[1][0] == 3


# ---- current block: invariants ----------------------------------------------
def test_delta_is_drift_minus_numpy_mean_of_earlier_steps():
    rng = np.random.default_rng(7)
    Ds = rng.exponential(0.3, size=40).astype(np.float32)
    out, hs, hn = _run_history(list(Ds), 0.3, 2.0, 0.9)
    for t in range(1, len(Ds)):
        want = float(Ds[t]) - np.mean(Ds[:t].astype(np.float64))
        assert out[t][1] == pytest.approx(want, rel=1e-6, abs=1e-7)
    assert hn[0] == len(Ds)
    assert hs[0, 0] == pytest.approx(np.sum(Ds.astype(np.float64)), rel=1e-14)


def test_drift_commits_shrink_as_alpha_grows():
    rng = np.random.default_rng(11)
    W, Nb, T = 3, 16, 6
    s = O.Shape(W=W, N=Nb + 4, d=16, Nb=Nb, K=1)
    Ds = rng.exponential(0.5, size=(T, W, Nb)).astype(np.float32)
    conf = rng.uniform(0, 1, size=(W, Nb + 4)).astype(np.float32)
    prev = None
    for alpha in (0.0, 0.5, 1.0, 4.0, 50.0):
        hs, hn = np.zeros((W, Nb)), np.zeros(W, np.int32)
        bits = []
        for t in range(T):
            r = O.commit_block(s, Ds[t], conf, 2, alpha, 0.8, hs, hn)
            bits.append(r["commit"] & 1)
        bits = np.stack(bits)
        if prev is not None:
            assert np.all(bits <= prev)
        prev = bits
    assert prev.sum() < bits.size


def test_windows_are_independent_and_block_offset_is_applied():
    rng = np.random.default_rng(3)
    W, N, Nb, b0 = 4, 12, 3, 5
    s = O.Shape(W=W, N=N, d=16, Nb=Nb, K=1)
    conf = rng.uniform(0, 1, size=(W, N)).astype(np.float32)
    D1 = rng.exponential(1.0, size=(W, Nb)).astype(np.float32)
    D2 = rng.exponential(1.0, size=(W, Nb)).astype(np.float32)
    hs, hn = np.zeros((W, Nb)), np.zeros(W, np.int32)
    O.commit_block(s, D1, conf, b0, 0.7, 0.6, hs, hn)
    full = O.commit_block(s, D2, conf, b0, 0.7, 0.6, hs, hn)
    for w in range(W):
        s1 = O.Shape(W=1, N=N, d=16, Nb=Nb, K=1)
        h1, n1 = np.zeros((1, Nb)), np.zeros(1, np.int32)
        O.commit_block(s1, D1[w:w + 1].copy(), conf[w:w + 1].copy(), b0, 0.7, 0.6, h1, n1)
        one = O.commit_block(s1, D2[w:w + 1].copy(), conf[w:w + 1].copy(), b0, 0.7, 0.6, h1, n1)
        assert np.array_equal(one["commit"][0], full["commit"][w])
        # the confidence bit reads window positions b0 .. b0+Nb-1
        assert np.array_equal((full["commit"][w] >> 1) & 1, (conf[w, b0:b0 + Nb] >= 0.6).astype(np.uint8))


def test_zero_count_starts_a_fresh_history():
    hs = np.full((1, 1), 123.0)
    out, hs, hn = [], hs, np.zeros(1, np.int32)
    r, hs, hn = _block([0.5], [0.0], 1.0, 0.9, hs, hn)
    assert hs[0, 0] == 0.5 and hn[0] == 1
    hn[0] = -3                     # a negative count also counts as none
    r, hs, hn = _block([0.25], [0.0], 1.0, 0.9, hs, hn)
    assert r["commit"][0, 0] == 0 and hs[0, 0] == 0.25 and hn[0] == 1


def test_nan_drift_never_commits_by_drift():
    out, hs, _ = _run_history([0.1, float("nan"), 5.0], 0.0, 0.0, 0.9)
    assert out[1][0] == 0 and out[2][0] == 0
    assert np.isnan(hs[0, 0])


@pytest.mark.parametrize("alpha,tau_s,b0", [(-1.0, 0.9, 0), (float("nan"), 0.9, 0),
                                            (1.0, float("inf"), 0), (1.0, 0.9, 7)])
def test_block_rejects_bad_arguments(alpha, tau_s, b0):
    s = O.Shape(W=1, N=8, d=16, Nb=2, K=1)
    with pytest.raises(O.OracleError):
        O.commit_block(s, np.zeros((1, 2), np.float32), np.zeros((1, 8), np.float32), b0, alpha,
                       tau_s, np.zeros((1, 2)), np.zeros(1, np.int32))


# ---- suffix block ----------------------------------------------------------------
def _suffix(assign, idx, b0, Nb, conf, tau_s, K):
    assign = np.atleast_2d(np.asarray(assign, np.int32))
    W, N = assign.shape
    idx = np.atleast_2d(np.asarray(idx, np.int32))
    s = O.Shape(W=W, N=N, d=16, Nb=Nb, K=K)
    return O.commit_suffix(s, assign, idx, idx.shape[1], b0, np.atleast_2d(
        np.asarray(conf, np.float32)), tau_s)


def test_suffix_worked_case():
    # N=10, block rows 4..5, suffix rows 6..9.
    # cluster 1 = rows {2,3,6,7,8}: 3 of 5 members in the suffix -> suffix cluster
    # cluster 2 = rows {4,5,9}: 1 of 3 -> not; cluster 0 = rows {0,1}: 0 of 2 -> not
    assign = [0, 0, 1, 1, 2, 2, 1, 1, 1, 2]
    conf = [0.99] * 6 + [0.5, 0.9, 0.95, 0.89]
    r = _suffix(assign, [2, 0], 4, 2, conf, 0.9, 3)
    assert r["flag"][0] == 0 and not r["commit"].any()
    r = _suffix(assign, [0, 1], 4, 2, conf, 0.9, 3)
    assert r["flag"][0] == 1
    # only suffix rows with conf >= 0.9 (0.9 itself included); block and prefix rows never
    assert r["commit"][0].tolist() == [0, 0, 0, 0, 0, 0, 0, 1, 1, 0]


def test_suffix_majority_is_strict_and_boundary_row_is_not_suffix():
    # cluster 0 = rows {3, 4, 6, 7}: rows 6, 7 are suffix (block 4..5) -> exactly
    # half -> not a suffix cluster
    assign = [1, 1, 1, 0, 0, 1, 0, 0]
    conf = [1.0] * 8
    assert _suffix(assign, [0], 4, 2, conf, 0.5, 2)["flag"][0] == 0
    # with the block at 3..4 the suffix starts at row 5: rows 6, 7 of {3,4,6,7}
    # are still half; moving row 4 into the suffix (block 2..3) makes 3 of 4
    assert _suffix(assign, [0], 3, 2, conf, 0.5, 2)["flag"][0] == 0
    assert _suffix(assign, [0], 2, 2, conf, 0.5, 2)["flag"][0] == 1


def test_suffix_invariants_random():
    rng = np.random.default_rng(5)
    W, N, Nb, K, k = 6, 64, 8, 8, 3
    assign = rng.integers(0, K, size=(W, N)).astype(np.int32)
    # make the first clusters mostly suffix in some windows
    assign[:3, 40:] = 0
    idx = np.stack([rng.permutation(K)[:k] for _ in range(W)]).astype(np.int32)
    idx[0, 0] = 0
    conf = rng.uniform(0, 1, size=(W, N)).astype(np.float32)
    b0 = 20
    r = _suffix(assign, idx, b0, Nb, conf, 0.6, K)
    assert r["flag"][0] == 1
    for w in range(W):
        c = r["commit"][w]
        assert not c[:b0 + Nb].any()
        if r["flag"][w]:
            assert np.array_equal(c[b0 + Nb:], (conf[w, b0 + Nb:] >= 0.6).astype(np.uint8))
        else:
            assert not c.any()
        # the order of the top-k list does not matter
        r2 = _suffix(assign[w], idx[w][::-1].copy(), b0, Nb, conf[w], 0.6, K)
        assert r2["flag"][0] == r["flag"][w]


def test_suffix_ignores_out_of_range_entries():
    assign = [0, 0, 5, -1, 0, 0]         # 5 and -1 are not clusters
    r = _suffix(assign, [7, -2], 0, 2, [1.0] * 6, 0.5, 2)
    assert r["flag"][0] == 0
    r = _suffix(assign, [7, 0], 0, 2, [1.0] * 6, 0.5, 2)
    # cluster 0 = rows {0,1,4,5}; suffix rows are 2..5 -> 2 of 4: not a majority
    assert r["flag"][0] == 0
    r = _suffix(assign, [0], 0, 1, [1.0] * 6, 0.5, 2)
    # suffix rows 1..5 -> rows {1,4,5} of {0,1,4,5}: 3 of 4
    assert r["flag"][0] == 1 and r["commit"][0].tolist() == [0, 1, 1, 1, 1, 1]


@pytest.mark.parametrize("k,b0,tau_s", [(0, 0, 0.5), (3, 0, 0.5), (1, 9, 0.5),
                                        (1, 0, float("nan"))])
def test_suffix_rejects_bad_arguments(k, b0, tau_s):
    s = O.Shape(W=1, N=10, d=16, Nb=2, K=2)
    with pytest.raises(O.OracleError):
        O.commit_suffix(s, np.zeros((1, 10), np.int32), np.zeros((1, max(k, 1)), np.int32), k, b0,
                        np.zeros((1, 10), np.float32), tau_s)
