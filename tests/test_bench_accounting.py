"""The benchmark's accounting, on the CPU: the algorithmic bytes and flops it
divides by the measured times (every input a kernel needs read once, every
output written once), the recorded-traffic lookup, and the refusal of more
than one GPU."""
import json
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402

CFG = synth.CONFIGS["llada8b-batch"]


def test_benchmark_workload_shape():
    assert (CFG.W, CFG.N, CFG.d, CFG.K, CFG.Hq, CFG.Hkv, CFG.dh, CFG.Nb, CFG.k, CFG.iters) == \
        (512, 1024, 4096, 64, 32, 32, 128, 32, 4, 8)
    assert CFG.bf16


def test_assign_pass_bytes_and_flops():
    W, N, d, K = CFG.W, CFG.N, CFG.d, CFG.K
    byts, flops = bench.kernel_work("k_assign_bf16<KB, NB, false>", CFG)
    assert byts == W * N * d * 2 + W * K * d * 2 + W * N * 4 == 4_565_499_904
    assert flops == 2 * W * N * K * d
    # arithmetic intensity K flop/B: under the bf16 ridge, so the HBM roofline applies
    assert flops / byts < bench.BF16_PEAK_TFLOPS * 1e12 / (bench.HBM_PEAK_GBS * 1e9)
    # the first pass reads the fp32 centres
    first, _ = bench.kernel_work("k_assign_bf16<KB, NB, true>", CFG)
    assert first == byts + W * K * d * 2
    # ... unless the launch is small and reads the bf16 copy
    small_first, _ = bench.kernel_work("k_assign_bf16<KB, NB, true>/bf16", CFG)
    assert small_first == byts


def test_coder_bytes():
    W, N, d, K = CFG.W, CFG.N, CFG.d, CFG.K
    byts, _ = bench.kernel_work("k_residual_grouped<T, BPL, FULL>", CFG)
    # H, fp32 centres, norm + assignment + row scale, E2M1 codes, E4M3 block scales
    assert byts == W * N * d * 2 + W * K * d * 4 + 3 * W * N * 4 + W * N * d // 2 + W * N * d // 16
    # the exact-path kernel codes a handful of listed rows: no full-pass figure
    assert bench.kernel_work("k_residual_listed<T, CPL>", CFG) is None


def test_coding_update_bytes():
    """The first update that also codes the rows: the update's bytes plus the
    codes and scales written; the rows are read once."""
    W, N, d, K = CFG.W, CFG.N, CFG.d, CFG.K
    upd, _ = bench.kernel_work("k_update<T, CH>", CFG)
    both, _ = bench.kernel_work("k_update_code<CH, BPL, FULL>", CFG)
    assert both - upd == W * N * d // 2 + W * N * d // 16 + W * N * 4
    coder, _ = bench.kernel_work("k_residual_grouped<T, BPL, FULL>", CFG)
    assert both < upd + coder          # neither the rows nor the centres read twice


def test_proxy_counts_the_previous_distribution():
    L = CFG.W * CFG.Hq * CFG.Nb * CFG.K
    q = CFG.W * CFG.Nb * CFG.Hq * CFG.dh * 2
    ck = CFG.W * CFG.K * CFG.Hkv * CFG.dh * 2
    for name in ("k_proxy_bf16<KB, NBQ>", "k_proxy_rows<NBQ>", "k_proxy_head<KB>"):
        byts, flops = bench.kernel_work(name, CFG)
        assert byts == q + ck + 2 * L * 4, name
        assert flops == 2.0 * CFG.W * CFG.Hq * CFG.Nb * CFG.K * CFG.dh
    # the score pass reads both distributions and the rows' drifts once
    byts, _ = bench.kernel_work("k_drift_scores", CFG)
    assert byts == 2 * L * 4 + CFG.W * CFG.Hq * CFG.Nb * 4 + CFG.W * (CFG.K + CFG.Nb) * 4


def test_gather_scales_with_the_rows_selected():
    assert bench.kernel_work("k_gather_rows<uint16_t>", CFG) is None     # rows unknown
    a, _ = bench.kernel_work("k_gather_rows<uint16_t>", CFG, 50.0)
    b, _ = bench.kernel_work("k_gather_rows<uint16_t>", CFG, 100.0)
    per_row = (b - a) / (50.0 * CFG.W)
    KV = CFG.Hkv * CFG.dh
    assert per_row == CFG.d // 2 + CFG.d // 16 + 16 + CFG.d * 2 + 4 * KV * 2


def test_recorded_traffic_is_tied_to_the_sources():
    c5 = synth.CONFIGS["llada8b-long"]
    # the coding update re-reads each cluster's rows after rebuilding its centre
    for name, cfg, lo, hi in (("k_assign_bf16<KB, NB, true>", CFG, 0.99, 1.05),
                              ("k_update_code<CH, BPL, FULL>", CFG, 1.0, 2.0),
                              ("k_assign_wide_dma<true>", c5, 0.99, 1.05),
                              ("k_update_code<CH, BPL, FULL>", c5, 1.0, 2.0),
                              ("k_keys<uint16_t>", c5, 0.99, 1.05)):
        got = bench.recorded_traffic(name, cfg.name)
        if got is not None:       # the committed counters match the committed kernel sources
            assert lo < got / bench.kernel_work(name, cfg)[0] < hi, name
        assert bench.recorded_traffic(name, "another-workload") is None
    assert bench.recorded_traffic("k_keys<uint16_t>", CFG.name) is None


def test_compulsory_work_matches_the_per_token_layer_figures():
    """The step's compulsory bytes per window-token-layer with the expected
    N k / K gathered rows: 25,245 B for the 1024-token windows (K = 64,
    k = 4) and 23,229 B for the 8192-token windows (K = 256, k = 16); flops
    iters * 2 K d + proxy attention."""
    for name, per_tok in (("llada8b-batch", 25_245), ("llada8b-long", 23_229)):
        cfg = synth.CONFIGS[name]
        M = cfg.N * cfg.k / cfg.K
        byts, flops = bench.compulsory_work(cfg, M)
        assert abs(byts / (cfg.W * cfg.N) - per_tok) < 1.0, (name, byts / (cfg.W * cfg.N))
        assert flops == cfg.W * (cfg.iters * 2.0 * cfg.N * cfg.K * cfg.d
                                 + 2.0 * cfg.Hq * cfg.Nb * cfg.K * cfg.dh)
    # the long window is flops-bound at the published peaks, the batch bytes-bound
    c5 = synth.CONFIGS["llada8b-long"]
    b5, f5 = bench.compulsory_work(c5, c5.N * c5.k / c5.K)
    assert f5 / (bench.BF16_PEAK_TFLOPS * 1e12) > b5 / (bench.HBM_PEAK_GBS * 1e9)
    c4 = synth.CONFIGS["llada8b-batch"]
    b4, f4 = bench.compulsory_work(c4, c4.N * c4.k / c4.K)
    assert f4 / (bench.BF16_PEAK_TFLOPS * 1e12) < b4 / (bench.HBM_PEAK_GBS * 1e9)


def test_headline_is_the_largest_single_gpu_workload():
    import inspect
    src = inspect.getsource(bench.main)
    assert 'default="llada8b-long"' in src
    c5 = synth.CONFIGS["llada8b-long"]
    assert (c5.W, c5.N, c5.d, c5.K, c5.k, c5.iters) == (128, 8192, 4096, 256, 16, 8)
    assert c5.name == "llada8b-32layers-4seq-N8192-K256"


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    msg = json.loads(p.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


@pytest.mark.parametrize("name", bench.CONFIG_NAMES)
def test_every_named_workload_exists(name):
    assert name in synth.CONFIGS
