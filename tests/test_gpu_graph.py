"""A step replayed from a HIP graph (DriftPath.step_graphed) must equal the
same step run eagerly, bit for bit, on every replay: the graphs of two input
sets are each replayed three times, with host copies and synchronisation (the
program's own eager work) between the replays."""
import sys

import numpy as np
import pytest
import torch

import synth
from parity_helpers import dev, host

pytestmark = pytest.mark.gpu

OUTPUTS = ("C", "assign", "counts", "row_norm", "Ck", "codes", "bscale", "rscale", "D_i",
           "score", "idx", "pos", "count", "H_hat", "K_out", "V_out", "commit_block",
           "commit_suffix", "suffix_flag", "hist_sum", "hist_n")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


CASES = [
    ("llada-4win", dict(W=4), "kl"),
    ("llada-4win-cosine", dict(W=4), "cosine"),
    ("k256-tile-kernel", dict(W=2, N=512, d=256, Hq=4, Hkv=4, dh=64, K=256, k=8), "kl"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_equal_eager_steps(case):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import drift_aware_kv_amd as P
    from drift_aware_kv_amd.pipeline import DriftPath, StepSpec
    P.lib()
    name, over, score = case
    cfg = synth.CONFIGS["llada8b-layer"].with_(**over)
    say("graph replay", name)
    spec = StepSpec(W=cfg.W, N=cfg.N, d=cfg.d, Hq=cfg.Hq, Hkv=cfg.Hkv, dh=cfg.dh, Nb=cfg.Nb,
                    K=cfg.K, k=cfg.k, iters=cfg.iters, bf16=True, softmax_scale=cfg.softmax_scale,
                    block_start=cfg.block_start, cluster_score=score)
    data = synth.generate(cfg)
    snaps = []
    for t in range(3):
        if t:
            synth.apply_drift(cfg, data, t)
        snaps.append([dev(data[k]) for k in ("H", "Kr", "V", "Q")] + [dev(synth.confidences(cfg, t))])
    order = [0, 1, 2, 1, 2, 1, 2]           # step t uses snapshot order[t]
    eager, graphed = DriftPath(spec), DriftPath(spec)
    for t, i in enumerate(order):
        eager.step(*snaps[i])
        graphed.step_graphed(*snaps[i])
        torch.cuda.synchronize()
        for o in OUTPUTS:
            a, b = host(getattr(eager, o)), host(getattr(graphed, o))
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"step {t}: {o}"
    assert len(graphed._graphs) == 2        # (snapshot 1, odd t) and (snapshot 2, even t)
