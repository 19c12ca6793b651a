"""GPU: the fit-and-code call (ps_kmeans_fit_nvfp4) against the two calls it
stands for, ps_kmeans_fit then ps_residual_nvfp4, bit for bit on every
output, over window formation and drift steps (rows moved between steps, so
later Lloyd updates rebuild some clusters and their rows are coded again),
on every thread layout of the coding update (1, 2 or 4 blocks of 16 per
lane, full rows and ragged ones), on the shapes that fall back to the coder
after the fit (fp32, rows longer than 4096), with rows the fast path
declines (zero rows, subnormal entries), clusters that lose every member and
clusters whose members are all zero rows (centres kept).
The two calls are themselves checked against the oracle elsewhere; the
pipeline's chained parity tests run the fit-and-code call against the
oracle."""
import sys

import numpy as np
import pytest
import torch

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


CASES = [
    # name, W, N, d, K, bf16
    ("k256-d4096", 2, 1100, 4096, 256, True),     # 4 blocks a lane, full rows, the LDS-fed tile kernel
    ("k64-d4096", 3, 700, 4096, 64, True),
    ("k128-d3584", 2, 600, 3584, 128, True),      # 4 blocks a lane, ragged rows
    ("k200-d2048", 2, 500, 2048, 200, True),      # 2 blocks a lane, full
    ("k37-d1024", 2, 400, 1024, 37, True),        # 1 block a lane, full
    ("k37-d80", 3, 300, 80, 37, True),            # 1 block a lane, ragged
    ("k20-d3072", 1, 300, 3072, 20, True),        # 4 blocks a lane, ragged, two update chunks
    ("k8-f32", 2, 200, 64, 8, False),             # fp32: the coder runs after the fit
    ("k70-d8192", 1, 300, 8192, 70, True),        # rows over 4096: the coder runs after the fit
    ("k256-w64", 64, 512, 256, 256, True),        # 16384 clusters: four per workgroup in the later updates
    ("k1-d48", 2, 130, 48, 1, True),              # one cluster: every row coded by one workgroup
]

OUTS = ("C", "a", "cnt", "rn", "Ck", "obj", "codes", "bsc", "rsc")


def _rows(rng, W, N, d, bf):
    H = rng.standard_normal((W, N, d)).astype(np.float32)
    H[0, 1] = 0.0                                  # zero row: listed for the exact coder
    H[0, 5] = 1e-40                                # subnormal entries: exact coder
    H[0, 5, 0] = 1.0
    return H


def _to_dtype(H, bf):
    """bf16 by round to nearest even (finite inputs), or the fp32 rows as they are."""
    if not bf:
        return H
    u = np.ascontiguousarray(H, dtype=np.float32).view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


# every shape with the default fixed-point exit, two with every pass in full
RUNS = [(c, 0) for c in CASES] + [(c, 2) for c in CASES if c[0] in ("k256-d4096", "k37-d80")]


@pytest.mark.parametrize("case,flags", RUNS,
                         ids=[c[0] + ("-all-passes" if f else "") for c, f in RUNS])
def test_fit_and_code_matches_the_two_calls(P, case, flags):
    name, W, N, d, K, bf = case
    say("fit and code", name, "flags", flags)
    rng = np.random.default_rng(5)
    dt = P.PS_BF16 if bf else P.PS_F32
    et = torch.bfloat16 if bf else torch.float32
    Hkv, dh = 2, 16
    s = P.Shape(W=W, N=N, d=d, Hq=2, Hkv=Hkv, dh=dh, Nb=1, K=K)
    H32 = _rows(rng, W, N, d, bf)
    Kr = _to_dtype(rng.standard_normal((W, N, Hkv, dh)).astype(np.float32), bf)

    def fresh():
        return dict(C=torch.zeros(W, K, d, device="cuda"),
                    a=torch.zeros(W, N, dtype=torch.int32, device="cuda"),
                    cnt=torch.zeros(W, K, dtype=torch.int32, device="cuda"),
                    rn=torch.zeros(W, N, device="cuda"),
                    Ck=torch.zeros(W, K, Hkv, dh, dtype=et, device="cuda"),
                    obj=torch.zeros(W, dtype=torch.float64, device="cuda"),
                    codes=torch.zeros(W, N, d // 2, dtype=torch.uint8, device="cuda"),
                    bsc=torch.zeros(W, N, d // 16, dtype=torch.uint8, device="cuda"),
                    rsc=torch.zeros(W, N, device="cuda"), ws=P.workspace(s, dt))

    A, B = fresh(), fresh()
    Krd = dev(Kr)
    for t in range(4):
        if t > 0:
            # drift: a tenth of the rows move by a large step, so the first
            # pass moves rows and later updates rebuild their clusters
            moved = rng.random((W, N)) < 0.1
            H32 = H32 + moved[..., None] * rng.standard_normal((W, N, d)).astype(np.float32) * 0.8
            H32[0, 1] = 0.0
        if t == 2:
            H32[1 % W, :, :] = H32[1 % W, :1, :]    # one window of identical rows: clusters lose every member
        if t == 1 and W >= 3:
            H32[2] = 0.0                           # a window of zero rows: members but no sum, centres kept
        Hd = dev(_to_dtype(H32, bf))
        init = P.PS_INIT_STRIDED if t == 0 else P.PS_INIT_GIVEN
        iters = 1 if t == 3 else 8                 # one iteration: only the coding update
        P.ps_kmeans_fit_nvfp4(s, dt, Hd, Krd, init, iters, A["C"], A["a"], A["cnt"], A["rn"], A["codes"],
                              A["bsc"], A["rsc"], A["Ck"], A["obj"], A["ws"], flags=flags)
        P.ps_kmeans_fit(s, dt, Hd, Krd, init, iters, B["C"], B["a"], B["cnt"], B["rn"], B["Ck"], B["obj"],
                        B["ws"], flags=flags)
        P.ps_residual_nvfp4(s, dt, Hd, B["rn"], B["C"], B["a"], B["codes"], B["bsc"], B["rsc"], B["ws"])
        torch.cuda.synchronize()
        for key in OUTS:
            x, y = host(A[key]), host(B[key])
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), (name, t, key)
