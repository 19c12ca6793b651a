"""The drift step on a side stream, beside GEMM work on another stream (the
pages' latency hiding, technical summary 2.C), must give bit-identical results
to the same step run alone on the current stream: every kernel of the library
runs on the stream it is given, and the step reads and writes only its own
buffers."""
import sys

import numpy as np
import pytest
import torch

import synth
from parity_helpers import dev, host

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


OUTPUTS = ("C", "assign", "counts", "row_norm", "Ck", "codes", "bscale", "rscale", "D_i",
           "score", "idx", "pos", "count", "H_hat", "K_out", "V_out", "commit_block",
           "commit_suffix", "suffix_flag", "hist_sum")


def test_step_on_side_stream_beside_gemms_is_bit_identical():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import drift_aware_kv_amd as P
    from drift_aware_kv_amd.pipeline import DriftPath, StepSpec
    P.lib()
    cfg = synth.CONFIGS["llada8b-layer"].with_(W=8)
    spec = StepSpec(W=cfg.W, N=cfg.N, d=cfg.d, Hq=cfg.Hq, Hkv=cfg.Hkv, dh=cfg.dh, Nb=cfg.Nb,
                    K=cfg.K, k=cfg.k, iters=cfg.iters, bf16=True, softmax_scale=cfg.softmax_scale,
                    block_start=cfg.block_start)
    data = synth.generate(cfg)
    steps = []
    for t in range(3):
        if t:
            synth.apply_drift(cfg, data, t)
        steps.append([dev(data[k]) for k in ("H", "Kr", "V", "Q")] + [dev(synth.confidences(cfg, t))])
    torch.cuda.synchronize()

    say("reference run on the current stream")
    ref = DriftPath(spec)
    for ins in steps:
        ref.step(*ins)
    torch.cuda.synchronize()

    say("side-stream run beside GEMMs")
    side = DriftPath(spec)
    s_drift, s_gemm = torch.cuda.Stream(), torch.cuda.Stream()
    g = torch.Generator(device="cuda").manual_seed(3)
    A = torch.randn((4096, 4096), generator=g, device="cuda").to(torch.bfloat16)
    B = torch.randn((4096, 4096), generator=g, device="cuda").to(torch.bfloat16)
    torch.cuda.synchronize()
    for ins in steps:
        with torch.cuda.stream(s_gemm):
            for _ in range(8):
                A = (A @ B) * (1.0 / 64.0)
        with torch.cuda.stream(s_drift):
            side.step(*ins, stream=s_drift)
    torch.cuda.synchronize()
    for name in OUTPUTS:
        a, b = host(getattr(ref, name)), host(getattr(side, name))
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), name
