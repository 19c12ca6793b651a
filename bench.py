#!/usr/bin/env python3
"""Benchmark of the Polestar-Cache drift-detection step on one MI355X.

A step is one pass of the whole path over one batch of W windows:
  spherical K-Means (warm start, `iters` Lloyd iterations) + centroid keys ->
  NVFP4 residuals -> proxy attention + KL drift + cluster scores ->
  top-k clusters -> refresh gather (positions, rebuilt hidden rows, K/V rows)
  -> Polestar-Commit's current-block and suffix-block rules.
Inputs are seeded synthetic tensors already resident in HBM (one snapshot per
denoising step, generated on the device before the timed region).

The headline workload is the long-window batch (LLaDA-8B shape, 32 layers x
4 sequences, N = 8192, K = 256): the largest workload that fits one GPU.  The
512-window LLaDA-8B batch (N = 1024, K = 64) is timed after it as a secondary
figure in the same line.

Prints one JSON line: metric, value (window-token-layers scored per second),
the roofline of the dominant kernel (its HIP-event average launch time over the
timed region against its algorithmic bytes), the step against the compulsory
bytes and flops of the method, and the CPU oracle timed on a bounded sample of
the same workload and the same input bytes.

  python bench.py [--steps K] [--warmup W] [--config llada8b-long] [--gpus 1]
"""
import argparse
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

METRIC = "window-token-layers drift-scored/sec per step at 1 GPU; % HBM/MFMA roofline"
UNIT = "window-token-layers/s"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
# the workloads of synth.CONFIGS (the long-window batch is the headline; the
# 512-window batch its secondary figure)
CONFIG_NAMES = ("tiny-planted", "llada8b-layer", "dream7b-layer", "llada8b-batch", "llada8b-long")


def kernel_work(name, cfg, gathered=None):
    """Algorithmic (bytes, flops) of ONE launch of a library kernel over all W
    windows: every input the kernel needs read once, every output written once.
    `gathered` is the mean number of rows the refresh gather selected per
    window (data-dependent: measured in the run)."""
    W, N, d, K = cfg.W, cfg.N, cfg.d, cfg.K
    e = 2 if cfg.bf16 else 4
    KV = cfg.Hkv * cfg.dh
    L = W * cfg.Hq * cfg.Nb * K
    if name.startswith("k_assign"):
        # H and the centres read, the assignment written (the fp64 norms of the
        # first pass are a by-product); the first pass of a call below 129
        # clusters reads the fp32 centres
        ce = 4 if (name.startswith("k_assign_bf16") and name.endswith("true>")) else e
        return W * N * d * e + W * K * d * ce + W * N * 4, 2.0 * W * N * K * d
    if name.startswith("k_update_code"):
        # the first update (every cluster rebuilt) and the NVFP4 codes and
        # scales of every row, coded against the new centres; the rows are
        # read once (coding re-reads them from the caches)
        return (W * N * d * e + 2 * W * N * 4 + W * K * d * (4 + e) + W * (K + 1) * 4
                + W * N * d // 2 + W * N * d // 16 + W * N * 4, W * N * d * 10.0)
    if name.startswith("k_update"):
        return W * N * d * e + 2 * W * N * 4 + W * K * d * (4 + e) + W * (K + 1) * 4, W * N * d * 2.0
    if name.startswith("k_code_stale"):
        # every cluster coded again (the kernel counts the clusters it codes):
        # rows, norms and centres read, codes and scales written
        return (W * N * d * e + 2 * W * N * 4 + W * K * d * 4 + W * (K + 1) * 4
                + W * N * d // 2 + W * N * d // 16 + W * N * 4, W * N * d * 8.0)
    if name.startswith("k_residual_grouped") or name.startswith("k_residual<"):
        return (W * N * d * e + W * K * d * 4 + 3 * W * N * 4 + W * N * d // 2 + W * N * d // 16,
                W * N * d * 8.0)
    if name.startswith("k_keys"):
        return W * N * KV * e + W * N * 4 + W * K * KV * e, W * N * KV * 1.0
    if name.startswith("k_proxy"):
        # Q and the keys read, log-probabilities written, and (after window
        # formation, for the drift: fused, or each row's drift in the
        # head-parallel form) the previous step's read
        return (W * cfg.Nb * cfg.Hq * cfg.dh * e + W * K * KV * e + 2 * L * 4,
                2.0 * W * cfg.Hq * cfg.Nb * K * cfg.dh)
    if name.startswith("k_drift_scores"):
        # both distributions and the rows' drifts read, scores and D_i written
        return 2 * L * 4 + W * cfg.Hq * cfg.Nb * 4 + W * (K + cfg.Nb) * 4, L * 4.0
    if name.startswith("k_drift_kl"):
        return 2 * L * 4 + W * (cfg.Hq * cfg.Nb + cfg.Nb + K) * 4, L * 4.0
    if name.startswith("k_bucket"):
        return 2 * W * N * 4 + W * (K + 1) * 4, 0.0
    if name.startswith("k_drift_cosine"):
        return 2 * W * K * d * 4 + W * K * 4, 2.0 * W * K * d
    if name.startswith("k_centres_to_bf16"):
        return W * K * d * (4 + 2), 0.0
    if name.startswith("k_group_rows"):
        return 2 * W * N * 4, 0.0
    if name.startswith("k_gather_select"):
        return W * N * 4 + W * cfg.k * 4 + (gathered or 0.0) * W * 4 + W * 4, 0.0
    if name.startswith("k_gather_rows") and gathered is not None:
        # per selected row: codes, block and row scales, norm, assignment and
        # position read, rebuilt row written, K and V rows read and written;
        # per window: the k selected centres read
        per_row = d // 2 + d // 16 + 4 * 4 + d * e + 4 * KV * e
        return gathered * W * per_row + W * cfg.k * d * 4, gathered * W * d * 4.0
    if name.startswith("k_commit_block"):
        Nb = cfg.Nb
        return W * Nb * (4 + 4 + 16 + 1 + 4) + W * 8, 0.0
    if name.startswith("k_commit_suffix"):
        return W * N * (4 + 4 + 1) + W * (cfg.k * 4 + 1), 0.0
    return None


def compulsory_work(cfg, gathered):
    """The method's compulsory (bytes, flops) of one step over all W windows:
    H and the key rows read once (the window's H reused across the Lloyd
    iterations), norms and assignments written, the fp32 centres read and
    written, the centroid keys written and read, NVFP4 codes and scales
    written, the queries read, the log-probabilities written and the previous
    step's read, and for each gathered row its codes read, the rebuilt row
    written and its K and V rows read and written; flops: iters * 2NKd for the
    assignment plus 2 Hq Nb K dh for proxy attention.  `gathered` is the mean
    number of rows the gather selected per window."""
    e = 2 if cfg.bf16 else 4
    N, d, K = cfg.N, cfg.d, cfg.K
    KV = cfg.Hkv * cfg.dh
    M = gathered
    per_window = (N * d * e + N * KV * e + 2 * N * 4 + 2 * K * d * 4 + 2 * K * KV * e
                  + N * d // 2 + N * d // 16 + N * 4 + cfg.Nb * cfg.Hq * cfg.dh * e
                  + 2 * cfg.Hq * cfg.Nb * K * 4
                  + M * (d // 2 + d // 16 + 4) + M * d * e + 4 * M * KV * e)
    flops = cfg.iters * 2.0 * N * K * d + 2.0 * cfg.Hq * cfg.Nb * K * cfg.dh
    return cfg.W * per_window, cfg.W * flops


PROFILES = os.path.join(HERE, "profiles")
CSRC = os.path.join(HERE, "drift_aware_kv_amd", "csrc")
DEFAULT_SOURCES = ("ps_kmeans.hip", "ps_common.h")


def kernel_source_hash(sources=DEFAULT_SOURCES):
    """SHA-256 of the given kernel source files (under csrc/), in order."""
    import hashlib
    h = hashlib.sha256()
    for f in sources:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()


def recorded_traffic(kernel_name, cfg_name):
    """HBM bytes per launch of a library kernel from the committed rocprofv3
    counter summaries (profiles/traffic_*.txt), if one was taken on the
    current text of the sources it names (`sources=`, default the K-Means
    source and the shared header), on this kernel and workload; else None."""
    import glob
    for path in sorted(glob.glob(os.path.join(PROFILES, "traffic_*.txt"))):
        try:
            kv = dict(l.strip().split("=", 1) for l in open(path) if "=" in l and not l.startswith("#"))
        except (OSError, ValueError):
            continue
        if kv.get("workload") != cfg_name or kv.get("kernel") != kernel_name:
            continue
        sources = tuple(x for x in kv.get("sources", ",".join(DEFAULT_SOURCES)).split(",") if x)
        try:
            if kv.get("source_sha256") != kernel_source_hash(sources):
                continue
        except OSError:
            continue
        return float(kv["traffic_bytes_per_launch"])
    return None


def copy_calibration():
    """A plain streaming kernel of known size for calibrating the FETCH_SIZE /
    WRITE_SIZE counters: an elementwise negation that reads 1 GiB and writes
    1 GiB per launch, three launches."""
    import torch
    a = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read_per_launch": 1 << 30, "copy_bytes_written_per_launch": 1 << 30}))


class StandInForward:
    """Stand-in for the dLLM forward pass the drift path runs beside: the
    projection and FFN GEMMs of LLaDA-8B (hidden 4096, MHA 32 x 128, FFN
    12288 with a gated SiLU) over `tokens` rows, for `layers` layers, bf16 on
    hipBLASLt through torch.  One layer's weights serve every layer (436 MB,
    larger than the last-level cache, so each layer still streams them from
    HBM).  No attention over the cache and no model weights: it only occupies
    the GPU the way a forward pass's GEMMs do."""

    def __init__(self, tokens, layers=32, d=4096, ffn=12288, seed=5):
        import torch
        g = torch.Generator(device="cuda").manual_seed(seed)

        def w(i, o):
            return (torch.randn((i, o), generator=g, device="cuda") * i ** -0.5).to(torch.bfloat16)

        self.layers = layers
        self.Wqkv, self.Wo = w(d, 3 * d), w(d, d)
        self.Wgu, self.Wd = w(d, 2 * ffn), w(ffn, d)
        self.x0 = torch.randn((tokens, d), generator=g, device="cuda").to(torch.bfloat16)
        self.ffn = ffn
        self.flops = 2.0 * layers * tokens * (d * 3 * d + d * d + d * 2 * ffn + ffn * d)

    def run(self):
        import torch
        x = self.x0
        for _ in range(self.layers):
            qkv = x @ self.Wqkv
            o = qkv[:, : x.shape[1]] @ self.Wo
            gu = x @ self.Wgu
            h = torch.nn.functional.silu(gu[:, : self.ffn]) * gu[:, self.ffn:]
            x = x + o + h @ self.Wd
        return x


def latency_hiding(path, wl, first_input, steps):
    """Time the stand-in forward alone, the drift step alone, and both at once
    on two streams of default priority (forward on one, drift step on the
    other); the part of the drift step the forward hides is
    1 - (t_both - t_forward) / t_drift."""
    import torch
    sequences = max(1, path.shape.W // 32)          # 32 layers per sequence
    fwd = StandInForward(tokens=sequences * path.shape.Nb)
    s_fwd, s_drift = torch.cuda.Stream(), torch.cuda.Stream()

    def timed(fn):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            fn(first_input + i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    def forward_only(i):
        with torch.cuda.stream(s_fwd):
            fwd.run()

    def drift_only(i):
        with torch.cuda.stream(s_drift):
            path.step(*wl.inputs(i), stream=s_drift)

    def both(i):
        with torch.cuda.stream(s_fwd):
            fwd.run()
        with torch.cuda.stream(s_drift):
            path.step(*wl.inputs(i), stream=s_drift)

    forward_only(0)
    torch.cuda.synchronize()
    t_f = timed(forward_only)
    t_d = timed(drift_only)
    t_b = timed(both)
    exposed = max(t_b - t_f, 0.0)
    return {"forward": "LLaDA-8B projection + FFN GEMMs (hidden 4096, FFN 12288), 32 layers, "
                       f"{fwd.x0.shape[0]} tokens (the decode blocks of the batch's sequences), bf16",
            "forward_ms": t_f * 1e3, "forward_tflops": fwd.flops / t_f / 1e12,
            "drift_ms": t_d * 1e3, "both_ms": t_b * 1e3, "exposed_drift_ms": exposed * 1e3,
            "hidden_fraction": 1.0 - exposed / t_d, "steps": steps}


def ceilings():
    """Practical ceilings on this GPU, measured with torch's own kernels: HBM
    streaming as an elementwise copy of 4 GiB (read + write bytes counted) and a
    large bf16 GEMM (hipBLASLt) for the matrix cores."""
    import torch
    n = 1 << 31
    a = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    m = 8192
    x = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    y = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    z = torch.empty(m, m, device="cuda", dtype=torch.bfloat16)
    out = {}
    for name, fn, work, unit in (("hbm_copy", lambda: torch.neg(a, out=b), 4 * n, "GBs"),
                                 ("bf16_gemm", lambda: torch.matmul(x, y, out=z), 2 * m ** 3, "TFLOPs")):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            fn()
        e1.record()
        torch.cuda.synchronize()
        rate = work * 10 / (e0.elapsed_time(e1) * 1e-3)
        out[f"{name}_{unit}"] = rate / (1e9 if unit == "GBs" else 1e12)
    del a, b, x, y, z
    torch.cuda.empty_cache()
    return out


def bandwidth():
    print(json.dumps(ceilings()))


def cpu_threads():
    """Host threads for the oracle baseline: the cores this process may run
    on, at most 16 (the host share of one GPU on the benchmark machines)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def sample_windows(cfg, wl, n):
    """Host copies of n windows, spread over the batch, of the device inputs of
    step 0 (window formation) and step 1: the same bytes the GPU ran on."""
    import numpy as np
    import torch

    def host(t):
        t = t.detach()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        return t.cpu().numpy()

    ws = sorted({min(cfg.W - 1, (i * cfg.W) // n) for i in range(n)})
    out = []
    for w in ws:
        snaps = []
        for step in (0, 1):
            H, Kr, V, Q, conf = wl.inputs(step)
            snaps.append({k: np.ascontiguousarray(host(x[w:w + 1]))
                          for k, x in (("H", H), ("Kr", Kr), ("V", V), ("Q", Q), ("conf", conf))})
        out.append((w, snaps))
    return out


def cpu_baseline(cfg, samples, alpha, tau_s):
    """The oracle, unchanged, on a bounded sample of the workload: for each
    sampled window (the device's own input bytes), window formation at step 0
    (untimed) and then one steady-state step at step 1 (timed): warm-started
    K-Means, residuals, proxy attention + KL, top-k, gather, commit rules.
    One window per host thread, all threads started together (ctypes releases
    the interpreter lock inside the oracle)."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    import oracle as O

    s = O.Shape(W=1, N=cfg.N, d=cfg.d, Hq=cfg.Hq, Hkv=cfg.Hkv, dh=cfg.dh, Nb=cfg.Nb, K=cfg.K)
    dt = O.BF16 if cfg.bf16 else O.F32

    def prepare(sample):
        _, (s0, _) = sample
        init = O.INIT_FARTHEST if cfg.init0 == "farthest" else O.INIT_STRIDED
        ck0 = np.zeros((1, cfg.K, cfg.Hkv, cfg.dh), np.uint16 if cfg.bf16 else np.float32)
        r = O.kmeans_fit(s, dt, s0["H"], s0["Kr"], init, cfg.iters,
                         np.zeros((1, cfg.K, cfg.d), np.float32), ck0)
        lp = O.proxy_attn(s, dt, s0["Q"], r["Ck"], cfg.softmax_scale)["logp"]
        return r["C"], r["Ck"], lp

    def step(args):
        (_, (_, x)), (C, Ck, lp) = args
        hist_sum, hist_n = np.zeros((1, cfg.Nb)), np.zeros(1, np.int32)
        t0 = time.perf_counter()
        r = O.kmeans_fit(s, dt, x["H"], x["Kr"], O.INIT_GIVEN, cfg.iters, C.copy(), Ck.copy())
        q = O.residual_nvfp4(s, dt, x["H"], r["row_norm"], r["C"], r["assign"])
        pa = O.proxy_attn(s, dt, x["Q"], r["Ck"], cfg.softmax_scale, lp)
        tk = O.topk_clusters(s, pa["score"], cfg.k)
        O.refresh_gather(s, dt, r["assign"], tk["idx"], cfg.k, cfg.N, q["codes"], q["bscale"],
                         q["rscale"], r["C"], r["row_norm"], True, x["Kr"], x["V"])
        O.commit_block(s, pa["D_i"], x["conf"], cfg.block_start, alpha, tau_s, hist_sum, hist_n)
        O.commit_suffix(s, r["assign"], tk["idx"], cfg.k, cfg.block_start, x["conf"], tau_s)
        return time.perf_counter() - t0

    n = len(samples)
    with ThreadPoolExecutor(max_workers=n) as ex:
        p0 = time.perf_counter()
        states = list(ex.map(prepare, samples))
        prep = time.perf_counter() - p0
        t0 = time.perf_counter()
        times = list(ex.map(step, zip(samples, states)))
        wall = time.perf_counter() - t0
    times.sort()
    med = times[len(times) // 2]
    return {"value": n * cfg.N / wall, "unit": UNIT, "cores": n, "kind": "oracle",
            "sample": f"{n} windows (of {cfg.W}: {', '.join(str(w) for w, _ in samples)}) x 1 steady-state "
                      f"step (step 1, warm-started from an untimed formation at step 0, on the device's "
                      f"own input bytes of those steps) of {cfg.name} (N={cfg.N}, d={cfg.d}, K={cfg.K}, "
                      f"{cfg.iters} Lloyd iterations), one window per thread on {n} threads started together",
            "value_per_core": cfg.N / med,
            "per_core_note": "one thread's own window-step time (median over the threads) while all "
                             f"{n} run: the 1-core rate",
            "step_s": {"median": med, "min": times[0], "max": times[-1]},
            "wall_s": wall, "formation_s": prep}


def timed_steps(path, wl, first, steps, profile, max_launches=0):
    """Run steps first .. first+steps-1 between a synchronisation on each side;
    returns (elapsed seconds, sorted per-step HIP-event ms, kernel timer
    summary or {})."""
    import torch
    import drift_aware_kv_amd as P
    if profile:
        P.profile_begin(max_launches)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    marks[0].record()
    for i in range(first, first + steps):
        path.step(*wl.inputs(i))
        marks[i - first + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_ms = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(steps))
    prof = {}
    if profile:
        P.profile_end()
        prof = P.profile_summary()
    return t1 - t0, step_ms, prof


def kernel_figures(cfg, prof, steps, gathered, ms_per_step):
    """Per-kernel table, the dominant kernel's roofline and the whole step's
    figures against the compulsory work, from the kernel timer's summary of
    the timed steps."""
    kernels = {k: v for k, v in prof.items() if not k.startswith("#")}

    def done(v):
        """Part of its launches' work a kernel did: the Lloyd passes skip the
        windows at a fixed point and count the tiles they process."""
        return v[4] / v[5] if len(v) > 5 and v[5] else 1.0

    breakdown = {}
    for k, v in sorted(kernels.items(), key=lambda kv: -kv[1][1]):
        breakdown[k] = {"launches": v[0], "avg_ms": v[1] / v[0], "total_ms_per_step": v[1] / steps}
        if len(v) > 5 and v[5]:
            breakdown[k]["work_fraction"] = done(v)
        work = kernel_work(k, cfg, gathered)
        if work:   # scaled by the part of the work done (the later updates re-sum changed clusters only)
            breakdown[k]["algorithmic_GB_per_launch"] = work[0] * done(v) / 1e9
            breakdown[k]["achieved_GBs"] = work[0] * done(v) / (v[1] / v[0] * 1e-3) / 1e9
    roof = None
    if kernels:
        name, v = max(kernels.items(), key=lambda kv: kv[1][1])
        n, tot = v[0], v[1]
        work = kernel_work(name, cfg, gathered)
        avg_s = tot / n / 1e3
        if work:
            byts, flops = work[0] * done(v), work[1] * done(v)
            ai = flops / byts
            if ai > BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
                ach = flops / avg_s / 1e12
                roof = {"kernel": name, "bound": "mfma", "achieved": ach, "peak": BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": ach / BF16_PEAK_TFLOPS, "traffic": None}
            else:
                ach = byts / avg_s / 1e9
                roof = {"kernel": name, "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": ach / HBM_PEAK_GBS, "traffic": None}
            roof.update({"algorithmic_bytes_per_launch": byts, "flops_per_launch": flops,
                         "avg_launch_ms": avg_s * 1e3, "launches": n, "work_fraction": done(v),
                         "mfma_frac": flops / avg_s / 1e12 / BF16_PEAK_TFLOPS})
            # the counters were taken with every launch doing its full work
            roof["traffic"] = recorded_traffic(name, cfg.name) if done(v) == 1.0 else None
    # the whole step against the method's compulsory bytes and flops (H read
    # once per step); the bytes the kernels move by their own accounting (H
    # streamed once per Lloyd pass, by the coder, ...) are given beside it
    # (with the fixed-point exit the flops are those of the passes that ran,
    # counted by the Lloyd kernels, not the full iters x 2NKd)
    cb, cf = compulsory_work(cfg, gathered)
    t = ms_per_step * 1e-3
    moved, ran = 0.0, 0.0
    for kname, v in kernels.items():
        work = kernel_work(kname, cfg, gathered)
        if work:
            moved += work[0] * v[0] * done(v)
            if kname.startswith("k_assign") or kname.startswith("k_proxy"):
                ran += work[1] * v[0] * done(v)
    ran = ran / steps if kernels else cf
    hbm, mfma = cb / t / 1e9 / HBM_PEAK_GBS, ran / t / 1e12 / BF16_PEAK_TFLOPS
    t_roof = max(ran / (BF16_PEAK_TFLOPS * 1e12), cb / (HBM_PEAK_GBS * 1e9))
    step_roof = {"compulsory_bytes_per_step": cb, "compulsory_flops_per_step": cf,
                 "executed_flops_per_step": ran,
                 "bound": "mfma" if ran / (BF16_PEAK_TFLOPS * 1e12) > cb / (HBM_PEAK_GBS * 1e9) else "hbm",
                 "hbm_frac": hbm, "mfma_frac": mfma, "frac": t_roof / t,
                 "roofline_ms_per_step": 1e3 * t_roof,
                 "kernel_bytes_per_step": moved / steps if kernels else None}
    return roof, step_roof, breakdown


def make_path(cfg, args):
    from drift_aware_kv_amd.pipeline import DriftPath, StepSpec
    spec = StepSpec(W=cfg.W, N=cfg.N, d=cfg.d, Hq=cfg.Hq, Hkv=cfg.Hkv, dh=cfg.dh, Nb=cfg.Nb,
                    K=cfg.K, k=cfg.k, iters=cfg.iters, bf16=cfg.bf16, init0=cfg.init0,
                    softmax_scale=cfg.softmax_scale, cap=cfg.N, block_start=cfg.block_start,
                    cluster_score=args.cluster_score, residual_store=args.residual_store)
    return DriftPath(spec)


def load_workload(cfg, total):
    import torch
    from synth.device import DeviceWorkload
    free = torch.cuda.mem_get_info()[0]
    snap = DeviceWorkload.snapshot_bytes(cfg)
    out_bytes = 3 * snap  # gather outputs at cap = N, plus state: generous
    n_snap = max(2, min(total, int((0.6 * free - out_bytes) // snap)))
    print(f"[bench] {cfg.name}: generating {n_snap} input snapshots of {snap / 2**30:.1f} GiB",
          file=sys.stderr, flush=True)
    return DeviceWorkload(cfg, n_snap), n_snap


def secondary_workload(name, args):
    """The same measurement, shorter, on another workload: value, step time,
    the dominant kernel's roofline and the step against the compulsory work."""
    import torch
    import synth
    cfg = synth.CONFIGS[name]
    warm = 2
    wl, n_snap = load_workload(cfg, warm + args.steps)
    path = make_path(cfg, args)
    for i in range(warm):
        path.step(*wl.inputs(i))
    elapsed, step_ms, prof = timed_steps(path, wl, warm, args.steps, True, 64 * args.steps * (cfg.iters + 8))
    ms = 1e3 * elapsed / args.steps
    gathered = float(torch.clamp(path.count, max=path.cap).double().mean().item())
    roof, step_roof, _ = kernel_figures(cfg, prof, args.steps, gathered, ms)
    print(f"[bench] secondary {cfg.name}: {ms:.3f} ms/step", file=sys.stderr, flush=True)
    out = {"workload": cfg.name, "windows": cfg.W, "window_tokens": cfg.N, "clusters": cfg.K,
           "top_k": cfg.k, "value": args.steps * cfg.W * cfg.N / elapsed, "ms_per_step": ms,
           "steps": args.steps, "warmup": warm,
           "step_ms": {"median": step_ms[len(step_ms) // 2], "min": step_ms[0], "max": step_ms[-1]},
           "roofline": roof, "step_roofline": step_roof, "gathered_rows_per_window": gathered}
    del path, wl
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="llada8b-long", choices=sorted(CONFIG_NAMES))
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="host threads (= sampled windows) for the CPU oracle baseline (0 = the cores "
                         "this process may use, at most 16)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the secondary figure on the 512-window LLaDA-8B batch")
    ap.add_argument("--no-profile", action="store_true", help="skip the per-kernel event timer")
    ap.add_argument("--no-all-passes", action="store_true",
                    help="skip the secondary timing with every Lloyd pass of every window run in full")
    ap.add_argument("--cluster-score", default="kl", choices=["kl", "cosine"],
                    help="rank clusters by drift share (the method) or by centre movement "
                         "(the cosine-dissimilarity variant)")
    ap.add_argument("--residual-store", default="device", choices=["device", "host"],
                    help="keep the NVFP4 residual store in HBM, or in pinned host memory as the "
                         "pages' CPU offload (copied out each step, selected rows fetched back)")
    ap.add_argument("--no-scoring-only", action="store_true",
                    help="skip the secondary timing of the scoring half of the step on fixed clusters")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the secondary timing of the same steps replayed from HIP graphs")
    ap.add_argument("--no-overlap", action="store_true",
                    help="skip the latency-hiding figure (drift step beside a stand-in forward)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB copy (counter calibration) and exit")
    ap.add_argument("--bandwidth", action="store_true",
                    help="only measure the practical HBM and bf16 GEMM ceilings and exit")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip measuring the practical HBM and bf16 GEMM ceilings")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.bandwidth:
        bandwidth()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this path runs on one GPU; windows are independent, so more GPUs "
                                   "would each run their own share of the windows with no "
                                   "communication; --gpus must be 1"}))
        sys.exit(2)
    if args.steps < 1 or args.warmup < 1:
        print("need --steps >= 1 and --warmup >= 1 (the first warmup step is window formation)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import drift_aware_kv_amd as P
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    P.lib()
    cfg = synth.CONFIGS[args.config]
    total = args.warmup + args.steps
    wl, n_snap = load_workload(cfg, total)
    path = make_path(cfg, args)
    spec = path.spec
    torch.cuda.synchronize()

    for i in range(args.warmup):
        path.step(*wl.inputs(i))
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    # the timed region: every kernel bracketed by the kernel timer's events
    elapsed, step_ms, prof = timed_steps(path, wl, args.warmup, args.steps, not args.no_profile,
                                         64 * args.steps * (cfg.iters + 8))
    ms_per_step = 1e3 * elapsed / args.steps
    value = args.steps * cfg.W * cfg.N / elapsed
    print(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step", file=sys.stderr, flush=True)
    # rows the refresh gather selected per window in the last timed step
    gathered = float(torch.clamp(path.count, max=spec.cap).double().mean().item())
    roof, step_roof, breakdown = kernel_figures(cfg, prof, args.steps, gathered, ms_per_step)
    nxt = total

    # the same number of steps again without the kernel timer (its events are
    # the only difference): how much the timer itself costs
    untimed = None
    if not args.no_profile:
        u_el, _, _ = timed_steps(path, wl, nxt, args.steps, False)
        nxt += args.steps
        untimed = {"ms_per_step": 1e3 * u_el / args.steps, "value": args.steps * cfg.W * cfg.N / u_el}

    # secondary figure: the same steps with every Lloyd pass of every window
    # run in full (the headline skips a window's passes after one that moves
    # no row; the results are bit-identical), with its own kernel table
    allp = None
    if not args.no_all_passes:
        path.spec.kmeans_flags = P.PS_KMEANS_ALL_PASSES
        a_el, a_ms, a_prof = timed_steps(path, wl, nxt, args.steps, not args.no_profile,
                                         64 * args.steps * (cfg.iters + 8))
        nxt += args.steps
        path.spec.kmeans_flags = P.PS_KMEANS_DEFAULT
        a_roof, a_step, a_kern = kernel_figures(cfg, a_prof, args.steps, gathered, 1e3 * a_el / args.steps)
        allp = {"value": args.steps * cfg.W * cfg.N / a_el, "ms_per_step": 1e3 * a_el / args.steps,
                "roofline": a_roof, "step_roofline": a_step,
                "kernels_ms_per_step": {k: v["total_ms_per_step"] for k, v in a_kern.items()}}
        print(f"[bench] every Lloyd pass in full: {allp['ms_per_step']:.3f} ms/step", file=sys.stderr, flush=True)

    # secondary figure: the same steps replayed from HIP graphs (one graph per
    # input snapshot and step parity, captured in two untimed passes)
    graphed = None
    if not args.no_graph and args.residual_store == "device":
        ins = [wl.inputs(i) for i in range(args.warmup, total)]
        for _ in range(2):
            for x in ins:
                path.step_graphed(*x)
        torch.cuda.synchronize()
        g0 = time.perf_counter()
        for x in ins:
            path.step_graphed(*x)
        torch.cuda.synchronize()
        g1 = time.perf_counter()
        graphed = {"value": args.steps * cfg.W * cfg.N / (g1 - g0), "ms_per_step": 1e3 * (g1 - g0) / args.steps,
                   "graphs": len(path._graphs)}
        path._graphs.clear()
        print(f"[bench] graph replay: {graphed['ms_per_step']:.3f} ms/step", file=sys.stderr, flush=True)

    # secondary figure: the scoring half only (proxy attention and drift,
    # top-k, gather, commit rules) on the clusters of the last clustered step
    scoring = None
    if not args.no_scoring_only and args.cluster_score == "kl":
        ins = [wl.inputs(i) for i in range(args.warmup, total)]
        path.step(*ins[0], recluster=False)
        torch.cuda.synchronize()
        s0 = time.perf_counter()
        for x in ins:
            path.step(*x, recluster=False)
        torch.cuda.synchronize()
        s1 = time.perf_counter()
        scoring = {"value": args.steps * cfg.W * cfg.N / (s1 - s0), "ms_per_step": 1e3 * (s1 - s0) / args.steps}
        print(f"[bench] scoring only: {scoring['ms_per_step']:.3f} ms/step", file=sys.stderr, flush=True)

    hiding = None
    if not args.no_overlap:
        print("[bench] latency hiding beside a stand-in forward", file=sys.stderr, flush=True)
        hiding = latency_hiding(path, wl, total + args.steps, args.steps)
        print(f"[bench] hidden fraction {hiding['hidden_fraction']:.3f}", file=sys.stderr, flush=True)

    # host copies of the sampled windows' inputs for the CPU baseline, then the
    # device memory goes to the secondary workload
    samples = None
    if not args.no_cpu:
        samples = sample_windows(cfg, wl, args.cpu_threads or cpu_threads())
    del path, wl
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    secondary = None
    if not args.no_secondary and args.config == "llada8b-long":
        secondary = secondary_workload("llada8b-batch", args)

    measured = None
    if not args.no_ceilings:
        measured = ceilings()
        if roof:
            key = "hbm_copy_GBs" if roof["unit"] == "GB/s" else "bf16_gemm_TFLOPs"
            measured["dominant_kernel_frac_of_measured"] = roof["achieved"] / measured[key]

    cpu = None
    if samples:
        print(f"[bench] CPU oracle baseline on {len(samples)} threads", file=sys.stderr, flush=True)
        cpu = cpu_baseline(cfg, samples, spec.alpha, spec.tau_s)
        print(f"[bench] CPU oracle: {cpu['step_s']['median']:.1f} s per window-step", file=sys.stderr,
              flush=True)

    line = {
        "metric": METRIC, "value": value, "unit": UNIT, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if cfg.bf16 else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "windows": cfg.W, "window_tokens": cfg.N, "hidden": cfg.d,
                   "q_heads": cfg.Hq, "kv_heads": cfg.Hkv, "head_dim": cfg.dh, "block": cfg.Nb,
                   "clusters": cfg.K, "top_k": cfg.k, "lloyd_iters": cfg.iters,
                   "lloyd_exit": "a window's passes after one that moves no row are skipped (results "
                                 "bit-identical to running every pass; all_lloyd_passes times that)",
                   "drift": f"{cfg.drift} {cfg.drift_frac:.0%} rows x {cfg.drift_mag}",
                   "cluster_score": args.cluster_score, "residual_store": args.residual_store,
                   "commit": {"alpha": spec.alpha, "tau_s": spec.tau_s,
                              "block_start": cfg.block_start},
                   "input_snapshots": n_snap, "parallelism": "single GPU"},
        "roofline": roof,
        "step_roofline": step_roof,
        "cpu_baseline": cpu,
        "secondary": secondary,
        "measured_ceilings": measured,
        "without_kernel_timer": untimed,
        "all_lloyd_passes": allp,
        "graph_replay": graphed,
        "scoring_only": scoring,
        "step_ms": {"median": step_ms[len(step_ms) // 2], "min": step_ms[0], "max": step_ms[-1]},
        "gathered_rows_per_window": gathered,
        "latency_hiding": hiding,
        "kernels": breakdown,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
