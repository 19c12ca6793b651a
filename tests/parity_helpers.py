"""Helpers shared by the GPU parity tests: host <-> device transfer, and the
comparison rules (bit-exact for integer/byte results except documented
near-ties; 1e-3 relative or 1e-5 absolute for floating-point results)."""
import numpy as np
import torch

import oracle as O

RTOL, ATOL = 1e-3, 1e-5
TIE_COS = 1e-6     # assignment near-tie: oracle fp64 gap on the cosine scale
TIE_TOPK = 1e-6    # top-k near-tie: |s_a - s_b| <= 1e-6 * max(1, |s|)


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    return torch.from_numpy(a).cuda()


def host(t):
    t = t.detach()
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16f(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def close(a, b, rtol=RTOL, atol=ATOL):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.all(np.abs(a - b) <= np.maximum(atol, rtol * np.abs(b)))


def max_rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b) / np.maximum(np.abs(b), 1e-30))) if a.size else 0.0


def assignment_mismatches(H, C_in, bf16, got, want, row_norm):
    """Rows where the two assignments differ, split into near-ties (the oracle's
    fp64 scores of the two clusters differ by <= TIE_COS on the cosine scale,
    with the centres rounded as the assignment step rounds them) and real
    disagreements.  H [N][d] (uint16 bf16 or fp32), C_in [K][d] the centres
    both sides assigned against."""
    bad = np.nonzero(got != want)[0]
    Hf = (bf16f(H) if bf16 else H).astype(np.float64)
    Cb = (bf16f(O.f32_to_bf16(C_in)) if bf16 else C_in).astype(np.float64)
    ties, real = [], []
    for j in bad:
        s1 = Hf[j] @ Cb[got[j]]
        s2 = Hf[j] @ Cb[want[j]]
        n = max(float(row_norm[j]), 1e-30)
        (ties if abs(s1 - s2) / n <= TIE_COS else real).append(int(j))
    return ties, real


def check_centre_properties(H, bf16, row_norm, assign, C, counts):
    """Properties of one window's K-Means result that hold whatever the other
    side computed, checked with plain numpy on the device's outputs: counts
    are the member counts of the assignment, every non-empty centre is a unit
    vector along the sum of its members' unit rows (cosine >= 1 - 1e-6).
    H [N][d], row_norm [N], assign [N], C [K][d], counts [K]."""
    K = C.shape[0]
    assert np.array_equal(counts, np.bincount(assign, minlength=K)[:K]), "counts vs assignment"
    Hf = (bf16f(H) if bf16 else H).astype(np.float64)
    n = row_norm.astype(np.float64)
    X = np.where(n[:, None] > 0, Hf / np.where(n > 0, n, 1.0)[:, None], 0.0)
    S = np.zeros((K, Hf.shape[1]))
    np.add.at(S, assign, X)
    Cd = C.astype(np.float64)
    for k in np.nonzero(counts)[0]:
        ns = np.linalg.norm(S[k])
        if ns == 0:
            continue
        assert abs(np.linalg.norm(Cd[k]) - 1.0) < 1e-6, f"centre {k} is not a unit vector"
        assert Cd[k] @ S[k] / ns >= 1.0 - 1e-6, f"centre {k} does not point along its members"


def topk_equivalent(score, got, want):
    """Top-k lists equal, or differ only where the scores swapped are within
    TIE_TOPK of each other (same score multiset up to near-ties)."""
    if np.array_equal(got, want):
        return True
    sg = np.sort(score[got])[::-1]
    sw = np.sort(score[want])[::-1]
    tol = TIE_TOPK * np.maximum(1.0, np.abs(sw))
    return bool(np.all(np.abs(sg - sw) <= tol))


def commit_block_mismatches(got, want, delta_want, conf, alpha, tau_s, d_err):
    """Current-block commit bits that differ between the two sides, split into
    near-threshold cases (the oracle's delta within d_err of its threshold
    alpha*(tau_s-c)^2, where d_err bounds the difference of the two sides'
    deltas given the drift tolerance) and real disagreements.  Bit 1 (the
    confidence rule) reads identical inputs and must always agree."""
    assert np.array_equal(got & 2, want & 2), "confidence rule"
    bad = np.nonzero((got & 1) != (want & 1))
    gap = np.float64(tau_s) - conf.astype(np.float64)
    thr = np.float64(alpha) * (gap * gap)
    near = np.abs(delta_want.astype(np.float64) - thr) <= d_err
    ties = [tuple(int(x) for x in ix) for ix in zip(*bad) if near[ix]]
    real = [tuple(int(x) for x in ix) for ix in zip(*bad) if not near[ix]]
    return ties, real
