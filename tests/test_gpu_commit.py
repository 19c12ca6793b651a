"""GPU parity of the Polestar-Commit calls against the oracle on the same
seeded inputs: bit-exact (commit bits, suffix flags, fp32 deltas and the fp64
history are all single IEEE operations in the same order on both sides)."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import synth
from parity_helpers import dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import drift_aware_kv_amd as P
    P.lib()
    return P


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def nz(t):
    """An empty tensor has no device address; hand the call a small buffer
    instead (it reads and writes nothing when the shape has no rows)."""
    return t if t.numel() else torch.zeros(16, dtype=t.dtype, device=t.device)


BLOCK_CASES = [
    # name, W, N, Nb, block_start, alpha, tau_s, steps
    ("llada-batch", 512, 1024, 32, 496, 0.02, 0.9, 5),
    ("ragged", 7, 300, 37, 263, 0.5, 0.8, 4),
    ("block-is-window", 3, 40, 40, 0, 0.0, 0.5, 3),
    ("long-block", 2, 5000, 1500, 1700, 1.0, 0.95, 3),
    ("no-rows", 4, 16, 0, 16, 0.1, 0.9, 2),
]


@pytest.mark.parametrize("case", BLOCK_CASES, ids=[c[0] for c in BLOCK_CASES])
def test_commit_block_bit_exact(P, case):
    name, W, N, Nb, b0, alpha, tau_s, steps = case
    say("commit block", name)
    s = P.Shape(W=W, N=N, d=16, Nb=Nb, K=1)
    so = O.Shape(W=W, N=N, d=16, Nb=Nb, K=1)
    seed = synth.BASE_SEED + W * 7 + N
    hs_o, hn_o = np.zeros((W, Nb)), np.zeros(W, np.int32)
    hs = torch.zeros(W, Nb, dtype=torch.float64, device="cuda")
    hn = torch.zeros(W, dtype=torch.int32, device="cuda")
    commit = torch.full((W, Nb), 255, dtype=torch.uint8, device="cuda")
    delta = torch.zeros(W, Nb, device="cuda")
    fired = 0
    for t in range(steps):
        D = synth.uniform((W, Nb), seed, 10 + t, lo=0.0, hi=0.05)
        conf = synth.uniform((W, N), seed, 50 + t)
        if Nb >= 4:
            D[0, 0] = np.nan                                   # never fires; poisons its history
            conf[0, b0 + 1] = np.float32(tau_s)                # confidence rule at equality
            conf[min(1, W - 1), b0 + 2] = np.nan
        if t == 2:
            hn_o[W - 1] = -2                                   # a reset window: fresh history
        hn.copy_(dev(hn_o))
        P.ps_commit_block(s, nz(dev(D)), dev(conf), b0, alpha, tau_s, nz(hs), hn, nz(commit),
                          nz(delta))
        torch.cuda.synchronize()
        r = O.commit_block(so, D, conf, b0, alpha, tau_s, hs_o, hn_o)
        assert np.array_equal(host(commit), r["commit"]), f"step {t}: commit bits"
        assert np.array_equal(host(delta).view(np.uint32), r["delta"].view(np.uint32)), "delta"
        assert np.array_equal(host(hs).view(np.uint64), hs_o.view(np.uint64)), "history sums"
        assert np.array_equal(host(hn), hn_o), "history counts"
        fired += int((r["commit"] & 1).sum())
    if Nb and alpha < 1.0:
        assert fired > 0, "the drift rule never fired: the case does not exercise it"


def test_commit_block_threshold_boundary(P):
    """Deltas exactly on the threshold (exact binary values) do not fire; one
    ulp above does."""
    W, N, Nb = 1, 8, 4
    s = P.Shape(W=W, N=N, d=16, Nb=Nb, K=1)
    so = O.Shape(W=W, N=N, d=16, Nb=Nb, K=1)
    conf = np.full((1, N), 0.25, np.float32)
    above = np.nextafter(np.float32(0.75), np.float32(1.0))
    Ds = [np.full((1, Nb), 0.5, np.float32), np.array([[0.75, above, 0.7, 1.0]], np.float32)]
    hs_o, hn_o = np.zeros((W, Nb)), np.zeros(W, np.int32)
    hs = torch.zeros(W, Nb, dtype=torch.float64, device="cuda")
    hn = torch.zeros(W, dtype=torch.int32, device="cuda")
    commit = torch.zeros(W, Nb, dtype=torch.uint8, device="cuda")
    for D in Ds:
        P.ps_commit_block(s, dev(D), dev(conf), 2, 1.0, 0.75, hs, hn, commit)
        torch.cuda.synchronize()
        r = O.commit_block(so, D, conf, 2, 1.0, 0.75, hs_o, hn_o)
        assert np.array_equal(host(commit), r["commit"])
    assert host(commit)[0].tolist() == [0, 1, 0, 1]


SUFFIX_CASES = [
    # name, W, N, Nb, block_start, K, k
    ("llada-batch", 512, 1024, 32, 496, 64, 4),
    ("long-window", 128, 8192, 32, 4080, 256, 16),
    ("ragged", 5, 301, 13, 200, 37, 5),
    ("k-max", 2, 2048, 32, 100, 1024, 64),
    ("k-equals-K", 3, 64, 8, 0, 6, 6),
    ("suffix-empty", 3, 64, 8, 56, 6, 2),
]


@pytest.mark.parametrize("case", SUFFIX_CASES, ids=[c[0] for c in SUFFIX_CASES])
def test_commit_suffix_bit_exact(P, case):
    name, W, N, Nb, b0, K, k = case
    say("commit suffix", name)
    rng = np.random.default_rng(N + K)
    assign = rng.integers(0, K, size=(W, N)).astype(np.int32)
    # half the windows: a band of suffix rows joins a few clusters
    first = b0 + Nb
    for w in range(0, W, 2):
        if first < N:
            assign[w, first:] = np.where(rng.random(N - first) < 0.7,
                                         rng.integers(0, max(1, K // 8), N - first), assign[w, first:])
    assign[0, 0] = -3                                       # counts for no cluster
    assign[-1, -1] = K + 5
    idx = np.stack([rng.permutation(K)[:k] for _ in range(W)]).astype(np.int32)
    if W > 2:
        idx[1, 0] = -1                                      # ignored entries
        idx[2, -1] = K
    conf = synth.uniform((W, N), synth.BASE_SEED, 77)
    conf[0, -1] = 0.9
    s = P.Shape(W=W, N=N, d=16, Nb=Nb, K=K)
    flag = torch.full((W,), 7, dtype=torch.uint8, device="cuda")
    commit = torch.full((W, N), 7, dtype=torch.uint8, device="cuda")
    P.ps_commit_suffix(s, dev(assign), dev(idx), k, b0, dev(conf), 0.9, flag, commit)
    torch.cuda.synchronize()
    r = O.commit_suffix(O.Shape(W=W, N=N, d=16, Nb=Nb, K=K), assign, idx, k, b0, conf, 0.9)
    assert np.array_equal(host(flag), r["flag"])
    assert np.array_equal(host(commit), r["commit"])
    say("  flagged windows:", int(r["flag"].sum()), "of", W)
