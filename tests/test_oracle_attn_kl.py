"""Pins of the oracle's proxy attention and drift KL: textbook attention in the
K = N special case, the two-point KL closed form, scipy's relative entropy,
Gibbs' inequality, exact zeros and the score decomposition invariants."""
import numpy as np
import pytest
from scipy.special import rel_entr, log_softmax

import oracle as O


def _bf16_to_f32(b):
    return (b.astype(np.uint32) << 16).view(np.float32)


def _logp(rng, W, Hq, Nb, K, spread=3.0):
    z = rng.standard_normal((W, Hq, Nb, K)) * spread
    return log_softmax(z, axis=-1).astype(np.float32)


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (6, 2)])
def test_k_equals_n_is_textbook_attention(Hq, Hkv):
    """With K = N, strided seeding and one iteration every row is its own
    cluster and Ck = Kr exactly, so proxy attention must equal plain scaled
    dot-product attention softmax(Q K^T / sqrt(dh)) over the window rows."""
    rng = np.random.default_rng(20)
    N, d, dh, Nb = 20, 32, 16, 5
    H = O.f32_to_bf16(rng.standard_normal((1, N, d)).astype(np.float32))
    Kr = O.f32_to_bf16(rng.standard_normal((1, N, Hkv, dh)).astype(np.float32))
    Q = O.f32_to_bf16(rng.standard_normal((1, Nb, Hq, dh)).astype(np.float32))
    s = O.Shape(W=1, N=N, d=d, Hq=Hq, Hkv=Hkv, dh=dh, Nb=Nb, K=N)
    r = O.kmeans_fit(s, O.BF16, H, Kr, O.INIT_STRIDED, 1, np.zeros((1, N, d), np.float32))
    assert np.array_equal(r["Ck"], Kr)
    sigma = float(np.float32(1 / np.sqrt(dh)))
    pa = O.proxy_attn(s, O.BF16, Q, r["Ck"], sigma)
    q = _bf16_to_f32(Q[0]).astype(np.float64)         # [Nb][Hq][dh]
    k = _bf16_to_f32(Kr[0]).astype(np.float64)        # [N][Hkv][dh]
    G = Hq // Hkv
    for h in range(Hq):
        logits = q[:, h, :] @ k[:, h // G, :].T * sigma   # [Nb][N]
        ref = np.exp(logits - logits.max(1, keepdims=True))
        ref /= ref.sum(1, keepdims=True)
        got = np.exp(pa["logp"][0, h].astype(np.float64))
        assert np.allclose(got, ref, rtol=1e-6, atol=1e-9)


def test_gqa_equals_replicated_heads():
    rng = np.random.default_rng(21)
    W, Nb, Hq, Hkv, dh, K = 2, 3, 8, 2, 16, 5
    Q = rng.standard_normal((W, Nb, Hq, dh)).astype(np.float32)
    Ck = rng.standard_normal((W, K, Hkv, dh)).astype(np.float32)
    Ck_rep = np.repeat(Ck, Hq // Hkv, axis=2).copy()  # head h uses KV head h // 4
    s1 = O.Shape(W=W, N=K, d=16, Hq=Hq, Hkv=Hkv, dh=dh, Nb=Nb, K=K)
    s2 = O.Shape(W=W, N=K, d=16, Hq=Hq, Hkv=Hq, dh=dh, Nb=Nb, K=K)
    a = O.proxy_attn(s1, O.F32, Q, Ck, 0.25)
    b = O.proxy_attn(s2, O.F32, Q, Ck_rep, 0.25)
    assert np.array_equal(a["logp"], b["logp"])


def test_logp_normalised():
    rng = np.random.default_rng(22)
    W, Nb, Hq, dh, K = 2, 4, 3, 32, 17
    Q = rng.standard_normal((W, Nb, Hq, dh)).astype(np.float32) * 4
    Ck = rng.standard_normal((W, K, Hq, dh)).astype(np.float32)
    s = O.Shape(W=W, N=K, d=16, Hq=Hq, Hkv=Hq, dh=dh, Nb=Nb, K=K)
    pa = O.proxy_attn(s, O.F32, Q, Ck, 1.0)
    assert np.allclose(np.exp(pa["logp"].astype(np.float64)).sum(-1), 1.0, atol=1e-6)
    assert np.all(pa["logp"] <= 0)
    # no previous step: drift and scores are zero
    assert not pa["D_i"].any() and not pa["score"].any() and not pa["D_hi"].any()


def test_kl_identical_is_exactly_zero():
    rng = np.random.default_rng(23)
    lp = _logp(rng, 2, 3, 4, 9)
    s = O.Shape(W=2, N=9, d=16, Hq=3, Nb=4, K=9)
    for kind in (O.SCORE_KL_SHARE, O.SCORE_KL_SHARE_ABS, O.SCORE_ATTN_WEIGHTED):
        r = O.drift_kl(s, lp, lp.copy(), kind)
        assert not r["D_hi"].any() and not r["D_i"].any() and not r["score"].any()


def test_kl_two_point_closed_form():
    """K = 2: KL((p,1-p) || (q,1-q)) = p ln(p/q) + (1-p) ln((1-p)/(1-q))."""
    rng = np.random.default_rng(24)
    n = 200
    p = rng.uniform(0.01, 0.99, n)
    q = rng.uniform(0.01, 0.99, n)
    lp = np.stack([np.log(p), np.log1p(-p)], -1).astype(np.float32).reshape(1, 1, n, 2)
    lq = np.stack([np.log(q), np.log1p(-q)], -1).astype(np.float32).reshape(1, 1, n, 2)
    s = O.Shape(W=1, N=2, d=16, Hq=1, Nb=n, K=2)
    r = O.drift_kl(s, lp, lq)
    # the closed form evaluated at the stored (fp32) distributions
    P = np.exp(lp.astype(np.float64))[0, 0]
    Qd = np.exp(lq.astype(np.float64))[0, 0]
    pp, qq = P[:, 0], Qd[:, 0]
    ref = pp * np.log(pp / qq) + P[:, 1] * np.log(P[:, 1] / Qd[:, 1])
    assert np.allclose(r["D_hi"][0, 0], ref, rtol=1e-6, atol=1e-7)
    # and at the exact inputs, within what fp32 storage allows
    exact = p * np.log(p / q) + (1 - p) * np.log((1 - p) / (1 - q))
    assert np.allclose(r["D_hi"][0, 0], exact, rtol=1e-5, atol=1e-6)


def test_kl_matches_scipy_and_gibbs():
    rng = np.random.default_rng(25)
    W, Hq, Nb, K = 3, 4, 6, 33
    a, b = _logp(rng, W, Hq, Nb, K), _logp(rng, W, Hq, Nb, K)
    s = O.Shape(W=W, N=K, d=16, Hq=Hq, Nb=Nb, K=K)
    r = O.drift_kl(s, a, b)
    P, Qd = np.exp(a.astype(np.float64)), np.exp(b.astype(np.float64))
    ref = rel_entr(P, Qd).sum(-1)
    # rel_entr uses the direct ratio; the oracle the stored log-probabilities
    assert np.allclose(r["D_hi"], ref, rtol=1e-5, atol=1e-6)
    assert np.all(r["D_hi"] >= -1e-6)
    assert np.allclose(r["D_i"], r["D_hi"].astype(np.float64).mean(1), rtol=1e-6, atol=1e-9)


def test_kl_direction_is_current_against_previous():
    """D = KL(A^t || A^{t-1}): swapping the two arguments changes the value
    for asymmetric pairs; the closed form fixes which is which."""
    p = np.array([0.9, 0.1])
    q = np.array([0.5, 0.5])
    lp = np.log(p).astype(np.float32).reshape(1, 1, 1, 2)
    lq = np.log(q).astype(np.float32).reshape(1, 1, 1, 2)
    s = O.Shape(W=1, N=2, d=16, Hq=1, Nb=1, K=2)
    fwd = O.drift_kl(s, lp, lq)["D_hi"][0, 0, 0]
    assert abs(fwd - (0.9 * np.log(0.9 / 0.5) + 0.1 * np.log(0.1 / 0.5))) < 1e-6
    assert abs(fwd - (0.5 * np.log(0.5 / 0.9) + 0.5 * np.log(0.5 / 0.1))) > 0.1


@pytest.mark.parametrize("kind", [O.SCORE_KL_SHARE, O.SCORE_ATTN_WEIGHTED])
def test_scores_decompose_the_drift(kind):
    """sum_k s_k = sum_i D_i for the additive share and for the
    attention-weighted score (sum_k p_k = 1)."""
    rng = np.random.default_rng(26)
    W, Hq, Nb, K = 2, 5, 7, 12
    a, b = _logp(rng, W, Hq, Nb, K), _logp(rng, W, Hq, Nb, K)
    s = O.Shape(W=W, N=K, d=16, Hq=Hq, Nb=Nb, K=K)
    r = O.drift_kl(s, a, b, kind)
    assert np.allclose(r["score"].astype(np.float64).sum(1), r["D_i"].astype(np.float64).sum(1),
                       rtol=1e-5, atol=1e-6)


def test_abs_score_bounds_share():
    rng = np.random.default_rng(27)
    a, b = _logp(rng, 1, 2, 3, 8), _logp(rng, 1, 2, 3, 8)
    s = O.Shape(W=1, N=8, d=16, Hq=2, Nb=3, K=8)
    sh = O.drift_kl(s, a, b, O.SCORE_KL_SHARE)["score"]
    ab = O.drift_kl(s, a, b, O.SCORE_KL_SHARE_ABS)["score"]
    assert np.all(ab >= np.abs(sh) - 1e-7) and np.all(ab >= 0)


def test_fused_equals_unfused():
    rng = np.random.default_rng(28)
    W, Nb, Hq, Hkv, dh, K = 2, 4, 4, 2, 16, 9
    Q = O.f32_to_bf16(rng.standard_normal((W, Nb, Hq, dh)).astype(np.float32))
    Ck = O.f32_to_bf16(rng.standard_normal((W, K, Hkv, dh)).astype(np.float32))
    prev = _logp(rng, W, Hq, Nb, K)
    s = O.Shape(W=W, N=K, d=16, Hq=Hq, Hkv=Hkv, dh=dh, Nb=Nb, K=K)
    fused = O.proxy_attn(s, O.BF16, Q, Ck, 0.25, logp_prev=prev)
    alone = O.proxy_attn(s, O.BF16, Q, Ck, 0.25)
    kl = O.drift_kl(s, alone["logp"], prev)
    assert np.array_equal(fused["logp"], alone["logp"])
    for key in ("D_hi", "D_i", "score"):
        assert np.array_equal(fused[key], kl[key])


# Hand-worked case for the two score kinds that the invariants above leave
# open: 2 heads x 2 block rows x K = 2, with distributions whose terms
# p (l - l') have opposite signs on the same cluster, so that an absolute
# value taken after the sum, or weights taken from the previous step, change
# the result.  [h][i] -> (current distribution p, previous distribution q).
_WORKED = {
    (0, 0): ((3 / 4, 1 / 4), (1 / 2, 1 / 2)),
    (0, 1): ((1 / 4, 3 / 4), (1 / 2, 1 / 2)),
    (1, 0): ((1 / 2, 1 / 2), (3 / 4, 1 / 4)),
    (1, 1): ((7 / 8, 1 / 8), (1 / 8, 7 / 8)),
}
_L = np.log
# the terms p_k ln(p_k / q_k) of each (head, row), worked out by hand
_TERMS = {
    (0, 0): (3 / 4 * _L(3 / 2), 1 / 4 * _L(1 / 2)),
    (0, 1): (1 / 4 * _L(1 / 2), 3 / 4 * _L(3 / 2)),
    (1, 0): (1 / 2 * _L(2 / 3), 1 / 2 * _L(2)),
    (1, 1): (7 / 8 * _L(7), 1 / 8 * _L(1 / 7)),
}


def _worked_inputs():
    cur = np.zeros((1, 2, 2, 2), np.float32)
    prev = np.zeros((1, 2, 2, 2), np.float32)
    for (h, i), (p, q) in _WORKED.items():
        cur[0, h, i] = np.log(p)
        prev[0, h, i] = np.log(q)
    return O.Shape(W=1, N=2, d=16, Hq=2, Nb=2, K=2), cur, prev


def test_worked_case_drift_per_head_and_token():
    """D_{h,i} is the sum of the row's two terms; D_i their mean over the two
    heads (values: 0.1308, 0.1308, 0.1438, 1.4594)."""
    s, cur, prev = _worked_inputs()
    r = O.drift_kl(s, cur, prev)
    D = {hi: t[0] + t[1] for hi, t in _TERMS.items()}
    assert abs(D[(0, 0)] - 0.130812) < 1e-6 and abs(D[(1, 1)] - 1.459433) < 1e-6
    for (h, i), v in D.items():
        assert abs(r["D_hi"][0, h, i] - v) < 1e-6
    for i in range(2):
        assert abs(r["D_i"][0, i] - (D[(0, i)] + D[(1, i)]) / 2) < 1e-6


def test_worked_case_share_and_abs_scores():
    """KL_SHARE: s_k = (1/Hq) sum_{h,i} term_k; KL_SHARE_ABS: the same sum of
    |term_k|.  Cluster 0 collects +0.3041, -0.1733, -0.2027 and +1.7027, so the
    two differ (0.8154 vs 1.1914), and an absolute value of the sum (0.8154)
    is caught."""
    s, cur, prev = _worked_inputs()
    share = O.drift_kl(s, cur, prev, O.SCORE_KL_SHARE)["score"][0]
    ab = O.drift_kl(s, cur, prev, O.SCORE_KL_SHARE_ABS)["score"][0]
    for k in range(2):
        want_share = sum(t[k] for t in _TERMS.values()) / 2
        want_abs = sum(abs(t[k]) for t in _TERMS.values()) / 2
        assert abs(share[k] - want_share) < 1e-6, (k, share[k], want_share)
        assert abs(ab[k] - want_abs) < 1e-6, (k, ab[k], want_abs)
    assert abs(ab[0] - 1.191395) < 1e-6 and abs(share[0] - 0.815375) < 1e-6
    assert abs(ab[1] - 0.533599) < 1e-6 and abs(share[1] - 0.117073) < 1e-6


def test_worked_case_attention_weighted_score():
    """ATTN_WEIGHTED: s_k = (1/Hq) sum_{h,i} p_{h,i,k} D_{h,i} with the CURRENT
    step's attention p; weights from the previous step would give 0.2106 and
    0.7219 instead of 0.7399 and 0.1926."""
    s, cur, prev = _worked_inputs()
    got = O.drift_kl(s, cur, prev, O.SCORE_ATTN_WEIGHTED)["score"][0]
    D = {hi: t[0] + t[1] for hi, t in _TERMS.items()}
    for k in range(2):
        want = sum(_WORKED[hi][0][k] * D[hi] for hi in D) / 2
        assert abs(got[k] - want) < 1e-6, (k, got[k], want)
    assert abs(got[0] - 0.739868) < 1e-6 and abs(got[1] - 0.192581) < 1e-6
