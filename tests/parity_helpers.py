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


def check_centres_from_assignment(so, dtype, H, row_norm, assign, C_gpu, counts_gpu):
    """The GPU's centres and counts must equal the oracle's update step run on
    the GPU's own assignment (bit for bit: same fp64 operations in the same
    order, up to the summation order of ||S||), and every non-empty centre
    must be a unit vector."""
    r = O.kmeans_update(so, dtype, H, row_norm, assign, C_gpu)
    assert np.array_equal(counts_gpu, r["counts"]), "counts from the assignment"
    diff = C_gpu.view(np.uint32) != r["C"].view(np.uint32)
    assert close(C_gpu, r["C"], 1e-6, 1e-7), f"centres from the assignment: {max_rel(C_gpu, r['C'])}"
    ne = counts_gpu > 0
    nrm = np.linalg.norm(C_gpu.astype(np.float64), axis=-1)
    assert np.all(np.abs(nrm[ne] - 1.0) < 1e-6), "non-empty centres must be unit vectors"
    return int(diff.sum())


def topk_equivalent(score, got, want):
    """Top-k lists equal, or differ only where the scores swapped are within
    TIE_TOPK of each other (same score multiset up to near-ties)."""
    if np.array_equal(got, want):
        return True
    sg = np.sort(score[got])[::-1]
    sw = np.sort(score[want])[::-1]
    tol = TIE_TOPK * np.maximum(1.0, np.abs(sw))
    return bool(np.all(np.abs(sg - sw) <= tol))
