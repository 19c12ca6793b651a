"""The allocation-free K-Means entry point (ps_kmeans_fit_static) against the
workspace call it mirrors (ps_kmeans_fit), through the C ABI: the same inputs
must give bit-identical assignments, counts, row norms, centres, centroid keys
and objectives.  Two shapes in a row, the second smaller than the first, so
the second call runs over scratch that still holds the first call's data; each
shape is fitted twice (seeded, then warm-started from its own centres)."""
import zlib

import numpy as np
import pytest
import torch

from parity_helpers import host

pytestmark = pytest.mark.gpu

# name, W, N, d, K, Hkv, dh: the first runs the LDS-fed 256-cluster tile
# kernel (about 6.3 MiB of scratch), the second a ragged shape on the
# small-K kernel
CASES = [("k256-tile", 3, 2048, 4096, 256, 8, 128), ("k37-ragged", 2, 300, 80, 37, 2, 24)]


@pytest.fixture(scope="module")
def P():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import drift_aware_kv_amd as P
    P.lib()
    return P


def _outputs(P, case):
    _, W, N, d, K, Hkv, dh = case
    f = lambda *shape, dt=torch.float32: torch.zeros(*shape, dtype=dt, device="cuda")
    return dict(C=f(W, K, d), assign=f(W, N, dt=torch.int32), counts=f(W, K, dt=torch.int32),
                row_norm=f(W, N), Ck=f(W, K, Hkv, dh, dt=torch.bfloat16), objective=f(W, dt=torch.float64))


def test_static_scratch_matches_the_workspace_call(P):
    for case in CASES:
        name, W, N, d, K, Hkv, dh = case
        print(f"no-alloc K-Means: {name} W={W} N={N} d={d} K={K}", flush=True)
        g = torch.Generator(device="cuda").manual_seed(zlib.crc32(name.encode()))
        H = torch.randn(W, N, d, generator=g, device="cuda").to(torch.bfloat16)
        Kr = torch.randn(W, N, Hkv, dh, generator=g, device="cuda").to(torch.bfloat16)
        s = P.Shape(W=W, N=N, d=d, Hq=Hkv, Hkv=Hkv, dh=dh, Nb=1, K=K)
        a, b = _outputs(P, case), _outputs(P, case)
        ws = P.workspace(s, P.PS_BF16)
        for init, iters in ((P.PS_INIT_STRIDED, 3), (P.PS_INIT_GIVEN, 2)):
            P.ps_kmeans_fit_static(s, P.PS_BF16, H, Kr, init, iters, a["C"], a["assign"], a["counts"],
                                   a["row_norm"], a["Ck"], a["objective"])
            P.ps_kmeans_fit(s, P.PS_BF16, H, Kr, init, iters, b["C"], b["assign"], b["counts"],
                            b["row_norm"], b["Ck"], b["objective"], ws)
            torch.cuda.synchronize()
            for key in a:
                x, y = host(a[key]), host(b[key])
                assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), (name, init, key)
        assert len(np.unique(host(a["assign"]))) > 1


def test_shape_beyond_the_static_scratch_is_refused(P):
    W, N, d, K = 512, 1024, 4096, 64        # 256 MiB of bf16 centres alone
    s = P.Shape(W=W, N=N, d=d, Hq=32, Hkv=32, dh=128, Nb=1, K=K)
    H = torch.zeros(W, N, d, dtype=torch.bfloat16, device="cuda")
    out = _outputs(P, ("big", W, N, d, K, 32, 128))
    with pytest.raises(P.PsError) as e:
        P.ps_kmeans_fit_static(s, P.PS_BF16, H, None, P.PS_INIT_STRIDED, 1, out["C"], out["assign"],
                               out["counts"], out["row_norm"])
    assert e.value.status == P.PS_ERR_SCRATCH_LIMIT
