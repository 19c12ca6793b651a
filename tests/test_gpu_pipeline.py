"""Chained end-to-end parity of whole steps (kmeans -> residual -> proxy
attention + drift -> top-k -> gather -> commit rules) against the oracle run
from the same seeded inputs, on the workloads of the benchmark: the tiny
planted case, a LLaDA-8B layer, a Dream-7B layer (GQA), and at full size the
512-window LLaDA-8B batch and the 128-window long-window batch on sampled
windows (every window is independent, so a sampled window's results depend on
its own data only; the other windows carry random data of the same shape).

Each side runs its own chain: the oracle never reads anything the device
computed.  Where the two sides assign a row differently, the step is replayed
one Lloyd iteration at a time on both sides, each from its own state, to find
the first iteration that differs; every row that differs there must be a
near-tie (oracle fp64 gap <= 1e-6 on the cosine scale) under the centres both
sides started that iteration from.  That window's chains would then
legitimately part, but for the committed seeds no chain does: the tests
require every sampled window to be compared in full at every step, codes,
scales and rebuilt rows bit for bit on every row."""
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle as O
import synth
from parity_helpers import (ATOL, RTOL, assignment_mismatches, check_centre_properties, close,
                            commit_block_mismatches, dev, host, max_rel, topk_equivalent)

pytestmark = pytest.mark.gpu

ALPHA, TAU_S = 0.02, 0.9     # commit parameters of these runs (the pages give no values)


@pytest.fixture(scope="module")
def P():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import drift_aware_kv_amd as P
    P.lib()
    return P


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def oshape(cfg, W=1):
    return O.Shape(W=W, N=cfg.N, d=cfg.d, Hq=cfg.Hq, Hkv=cfg.Hkv, dh=cfg.dh, Nb=cfg.Nb, K=cfg.K)


def oracle_step(cfg, st, data, conf, t, iters=None, cluster_score="kl", recluster=True):
    """One oracle step for one window; st carries the oracle's own C, Ck,
    logp and commit history between steps.  recluster=False keeps the last
    step's clusters, keys and residual codes and runs only the scoring half."""
    s = oshape(cfg)
    dt = O.BF16 if cfg.bf16 else O.F32
    iters = cfg.iters if iters is None else iters
    if t == 0:
        init = O.INIT_FARTHEST if cfg.init0 == "farthest" else O.INIT_STRIDED
        C = np.zeros((1, cfg.K, cfg.d), np.float32)
        Ck = np.zeros((1, cfg.K, cfg.Hkv, cfg.dh), np.uint16 if cfg.bf16 else np.float32)
        hist_sum, hist_n = np.zeros((1, cfg.Nb)), np.zeros(1, np.int32)
    else:
        init, C, Ck = O.INIT_GIVEN, st["C"].copy(), st["Ck"].copy()
        hist_sum, hist_n = st["hist_sum"].copy(), st["hist_n"].copy()
    if recluster:
        r = O.kmeans_fit(s, dt, data["H"], data["Kr"], init, iters, C, Ck)
        q = O.residual_nvfp4(s, dt, data["H"], r["row_norm"], r["C"], r["assign"])
    else:
        r = {key: st[key] for key in ("C", "Ck", "assign", "counts", "row_norm")}
        q = {key: st[key] for key in ("codes", "bscale", "rscale")}
    pa = O.proxy_attn(s, dt, data["Q"], r["Ck"], cfg.softmax_scale,
                      None if t == 0 else st["logp"])
    out = dict(C=r["C"], Ck=r["Ck"], assign=r["assign"], counts=r["counts"], row_norm=r["row_norm"],
               codes=q["codes"], bscale=q["bscale"], rscale=q["rscale"], logp=pa["logp"],
               D_i=pa["D_i"], D_hi=pa["D_hi"], score=pa["score"], hist_sum=hist_sum, hist_n=hist_n)
    if t > 0:
        rank = pa["score"]
        if cluster_score == "cosine":
            rank = O.drift_cosine(s, r["C"], st["C"])
            out.update(score_cos=rank)
        tk = O.topk_clusters(s, rank, cfg.k)
        g = O.refresh_gather(s, dt, r["assign"], tk["idx"], cfg.k, cfg.N, q["codes"], q["bscale"],
                             q["rscale"], r["C"], r["row_norm"], True, data["Kr"], data["V"])
        out.update(idx=tk["idx"], pos=g["pos"], count=g["count"], H_hat=g["H_hat"],
                   K_out=g["K_out"], V_out=g["V_out"])
        cb = O.commit_block(s, pa["D_i"], conf, cfg.block_start, ALPHA, TAU_S, hist_sum, hist_n)
        cs = O.commit_suffix(s, r["assign"], tk["idx"], cfg.k, cfg.block_start, conf, TAU_S)
        out.update(commit_block=cb["commit"], delta=cb["delta"], suffix_flag=cs["flag"],
                   commit_suffix=cs["commit"])
    return out


def gpu_snapshot(path, w, t):
    sl = slice(w, w + 1)
    o = dict(C=host(path.C[sl]), Ck=host(path.Ck[sl]), assign=host(path.assign[sl]),
             counts=host(path.counts[sl]), row_norm=host(path.row_norm[sl]),
             codes=host(path.codes[sl]), bscale=host(path.bscale[sl]), rscale=host(path.rscale[sl]),
             logp=host(path.logp[t & 1][sl]), D_i=host(path.D_i[sl]), D_hi=host(path.D_hi[sl]),
             score=host(path.score[sl]), hist_sum=host(path.hist_sum[sl]),
             hist_n=host(path.hist_n[sl]))
    if t > 0 and path.score_cos is not None:
        o.update(score_cos=host(path.score_cos[sl]))
    if t > 0:
        o.update(idx=host(path.idx[sl]), pos=host(path.pos[sl]), count=host(path.count[sl]),
                 H_hat=host(path.H_hat[sl]), K_out=host(path.K_out[sl]), V_out=host(path.V_out[sl]),
                 commit_block=host(path.commit_block[sl]), delta=host(path.delta[sl]),
                 suffix_flag=host(path.suffix_flag[sl]), commit_suffix=host(path.commit_suffix[sl]))
    return o


def compare_step(cfg, g, o, conf, t, d_hist):
    """Both sides assigned every row alike: compare everything else."""
    assert np.array_equal(g["counts"], o["counts"])
    assert close(g["C"], o["C"], 1e-6, 1e-7), f"centres {max_rel(g['C'], o['C'])}"
    assert np.array_equal(g["Ck"], o["Ck"]) if cfg.bf16 else close(g["Ck"], o["Ck"], 1e-6, 1e-7)
    assert max_rel(g["row_norm"], o["row_norm"]) <= 1.2e-7
    # the coder's inputs of a row are its norm and its centre: where both are
    # bit-identical on the two sides, the codes must be too
    a = o["assign"][0]
    same_c = np.all(g["C"][0].view(np.uint32) == o["C"][0].view(np.uint32), axis=-1)
    rows = same_c[a] & (g["row_norm"][0].view(np.uint32) == o["row_norm"][0].view(np.uint32))
    # both sides sum the same fp64 terms in the same order: on an intact chain
    # every row's coder inputs are bit-identical, and so must every code be
    assert rows.all(), f"{int((~rows).sum())} rows have coder inputs that differ in some bit"
    assert np.array_equal(g["codes"], o["codes"]), "codes"
    assert np.array_equal(g["bscale"], o["bscale"]), "block scales"
    assert np.array_equal(g["rscale"].view(np.uint32), o["rscale"].view(np.uint32)), "row scales"
    assert close(g["logp"], o["logp"]), f"logp {max_rel(g['logp'], o['logp'])}"
    if t == 0:
        assert not g["D_i"].any() and not g["score"].any()
        return
    assert close(g["D_i"], o["D_i"]) and close(g["D_hi"], o["D_hi"]) and close(g["score"], o["score"])
    rank = o["score"]
    if "score_cos" in o:
        # fp64 dot products summed in different orders (at most d * 2^-53 apart
        # for unit vectors), each rounded once to fp32
        diff = np.abs(g["score_cos"].astype(np.float64) - o["score_cos"])
        tol = np.spacing(np.abs(o["score_cos"])).astype(np.float64) + cfg.d * 2.0 ** -53
        assert np.all(diff <= tol), "cosine scores"
        rank = o["score_cos"]
    assert topk_equivalent(rank[0], g["idx"][0], o["idx"][0]), "top-k"
    assert int(g["hist_n"][0]) == int(o["hist_n"][0]) == t
    assert close(g["hist_sum"], o["hist_sum"], RTOL, ATOL * t)
    ties, real = commit_block_mismatches(g["commit_block"][0], o["commit_block"][0], o["delta"][0],
                                         conf[0, cfg.block_start:cfg.block_start + cfg.Nb],
                                         ALPHA, TAU_S, d_hist)
    assert not real, f"current-block commit: {len(real)} disagreements away from the threshold"
    if ties:
        say(f"    step {t}: {len(ties)} near-threshold commit rows")
    if not np.array_equal(g["idx"], o["idx"]):
        return                                  # equivalent near-tie selection: nothing more to compare
    m = int(o["count"][0])
    assert int(g["count"][0]) == m
    assert np.array_equal(g["pos"][0, :m], o["pos"][0, :m])
    assert np.array_equal(g["K_out"][0, :m], o["K_out"][0, :m])
    assert np.array_equal(g["V_out"][0, :m], o["V_out"][0, :m])
    view = np.uint16 if cfg.bf16 else np.uint32
    assert np.array_equal(g["H_hat"][0, :m].view(view), o["H_hat"][0, :m].view(view)), "rebuilt rows"
    assert np.array_equal(g["suffix_flag"], o["suffix_flag"]), "suffix flag"
    assert np.array_equal(g["commit_suffix"], o["commit_suffix"]), "suffix commit"


def replay_first_difference(P, cfg, data, C_gpu, Ck_gpu, ost, t):
    """Replay one step's K-Means one Lloyd iteration at a time on both sides,
    the device from its own centres before the step and the oracle from its
    own; return the near-tie rows at the first iteration whose assignments
    differ (asserting there is no real disagreement, and that one differs)."""
    s = P.Shape(W=1, N=cfg.N, d=cfg.d, Hq=cfg.Hq, Hkv=cfg.Hkv, dh=cfg.dh, Nb=cfg.Nb, K=cfg.K)
    dt = P.PS_BF16 if cfg.bf16 else P.PS_F32
    odt = O.BF16 if cfg.bf16 else O.F32
    C, Ck = dev(C_gpu), dev(Ck_gpu)
    a = torch.zeros(1, cfg.N, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(1, cfg.K, dtype=torch.int32, device="cuda")
    rn = torch.zeros(1, cfg.N, device="cuda")
    ws = P.workspace(s, dt)
    Hd, Krd = dev(data["H"]), dev(data["Kr"])
    seed = O.INIT_FARTHEST if cfg.init0 == "farthest" else O.INIT_STRIDED
    oC = np.zeros((1, cfg.K, cfg.d), np.float32) if t == 0 else ost["C"].copy()
    for it in range(cfg.iters):
        first = t == 0 and it == 0
        init = (P.PS_INIT_FARTHEST if cfg.init0 == "farthest" else P.PS_INIT_STRIDED) if first \
            else P.PS_INIT_GIVEN
        C_in = O.kmeans_init(oshape(cfg), odt, data["H"], seed) if first else oC.copy()
        P.ps_kmeans_fit(s, dt, Hd, Krd, init, 1, C, a, cnt, rn, Ck, None, ws)
        torch.cuda.synchronize()
        r = O.kmeans_fit(oshape(cfg), odt, data["H"], None, seed if first else O.INIT_GIVEN, 1,
                         oC.copy())
        ga = host(a)[0]
        if not np.array_equal(ga, r["assign"][0]):
            ties, real = assignment_mismatches(data["H"][0], C_in[0], cfg.bf16, ga, r["assign"][0],
                                               r["row_norm"][0])
            assert not real, f"step {t} iteration {it}: {len(real)} real disagreements"
            return ties
        assert close(host(C), r["C"], 1e-6, 1e-7)
        oC = r["C"]
    raise AssertionError(f"step {t}: the step's assignment differs but no replayed iteration does")


def run_chained(P, cfg, steps, windows=None, W=None, cluster_score="kl", residual_store="device",
                score_only_from=None):
    """GPU DriftPath over `steps` steps with the commit rules; the oracle runs
    its own chain for each sampled window.  From step score_only_from on, both
    sides keep their clusters and run only the scoring half.  Returns the
    number of windows whose chains parted at a near-tie (the tests require
    none for their seeds: every sampled window is compared at every step)."""
    from drift_aware_kv_amd.pipeline import DriftPath, StepSpec
    W = cfg.W if W is None else W
    windows = list(range(W)) if windows is None else windows
    spec = StepSpec(W=W, N=cfg.N, d=cfg.d, Hq=cfg.Hq, Hkv=cfg.Hkv, dh=cfg.dh, Nb=cfg.Nb, K=cfg.K,
                    k=cfg.k, iters=cfg.iters, bf16=cfg.bf16, init0=cfg.init0,
                    softmax_scale=cfg.softmax_scale, cap=cfg.N, block_start=cfg.block_start,
                    alpha=ALPHA, tau_s=TAU_S, cluster_score=cluster_score,
                    residual_store=residual_store)
    path = DriftPath(spec)
    et = torch.bfloat16 if cfg.bf16 else torch.float32
    # device inputs: sampled windows from the generator, the rest random
    host_data = {w: synth.generate(cfg, w0=w, Wc=1) for w in windows}
    g = torch.Generator(device="cuda").manual_seed(1)

    def fill(shape):
        return torch.randn(shape, device="cuda", generator=g).to(et)

    Hd = fill((W, cfg.N, cfg.d))
    Krd = fill((W, cfg.N, cfg.Hkv, cfg.dh))
    Vd = fill((W, cfg.N, cfg.Hkv, cfg.dh))
    Qd = fill((W, cfg.Nb, cfg.Hq, cfg.dh))
    confd = torch.rand((W, cfg.N), device="cuda", generator=g)

    def upload(w, conf):
        for key, dst in (("H", Hd), ("Kr", Krd), ("V", Vd), ("Q", Qd)):
            src = dev(host_data[w][key][0])
            dst[w].copy_(src.view(et) if cfg.bf16 else src)
        confd[w].copy_(dev(conf[0]))

    ost = {w: None for w in windows}
    parted = {}
    d_max = {w: 0.0 for w in windows}
    for t in range(steps):
        if t > 0:
            for w in windows:
                synth.apply_drift(cfg, host_data[w], t, w0=w)
            Hd.add_(fill(Hd.shape) * 0.01)  # unchecked windows drift too
        conf = {w: synth.confidences(cfg, t, w0=w, Wc=1) for w in windows}
        for w in windows:
            upload(w, conf[w])
        say(f"  {cfg.name} step {t}: GPU")
        prevC = {w: host(path.C[w:w + 1]).copy() for w in windows}
        prevCk = {w: host(path.Ck[w:w + 1]).copy() for w in windows}
        recluster = score_only_from is None or t < score_only_from
        path.step(Hd, Krd, Vd, Qd, conf=confd, recluster=recluster)
        torch.cuda.synchronize()
        live = [w for w in windows if w not in parted]
        say(f"  {cfg.name} step {t}: oracle windows {live}")
        # the oracle's windows are independent: one host thread each (the
        # oracle library releases the interpreter lock while it runs)
        with ThreadPoolExecutor(max_workers=max(1, min(len(live), 16))) as ex:
            ores = dict(zip(live, ex.map(
                lambda w: oracle_step(cfg, ost[w], host_data[w], conf[w], t, cluster_score=cluster_score,
                                      recluster=recluster), live)))
        for w in windows:
            gs = gpu_snapshot(path, w, t)
            if recluster:     # the clusters describe this step's rows
                check_centre_properties(host_data[w]["H"][0], cfg.bf16, gs["row_norm"][0],
                                        gs["assign"][0], gs["C"][0], gs["counts"][0])
            if w in parted:
                continue
            o = ores[w]
            if not np.array_equal(gs["assign"], o["assign"]):
                ties = replay_first_difference(P, cfg, host_data[w], prevC[w], prevCk[w], ost[w], t)
                say(f"    window {w} step {t}: chains part at {len(ties)} near-tie rows")
                parted[w] = t
                continue
            if t > 0:
                d_max[w] = max(d_max[w], float(np.abs(o["D_i"]).max()))
            # bound on |delta_gpu - delta_oracle|: the drift tolerance on the
            # current drift plus on the mean of the earlier ones
            d_err = 2.0 * max(ATOL, RTOL * d_max[w])
            compare_step(cfg, gs, o, conf[w], t, d_err)
            ost[w] = o
    return len(parted)


def test_tiny_planted_three_steps_exact(P):
    cfg = synth.CONFIGS["tiny-planted"]
    assert run_chained(P, cfg, steps=3) == 0


def test_llada_layer_chained(P):
    cfg = synth.CONFIGS["llada8b-layer"]
    assert run_chained(P, cfg, steps=4) == 0


def test_llada_layer_chained_cosine_score(P):
    """The same chain with clusters ranked by how far their centres moved."""
    cfg = synth.CONFIGS["llada8b-layer"].with_(W=4)
    assert run_chained(P, cfg, steps=3, cluster_score="cosine") == 0


def test_llada_layer_chained_host_residual_store(P):
    """The same chain with the residual store in pinned host memory: the gather
    fetches the selected rows across PCIe."""
    cfg = synth.CONFIGS["llada8b-layer"].with_(W=2)
    assert run_chained(P, cfg, steps=3, residual_store="host") == 0


def test_llada_layer_scoring_only_steps(P):
    """Two clustered steps, then two steps that keep the clusters, keys and
    residual codes and only score (proxy attention and drift, top-k, gather
    with the step's own K/V rows, commit rules)."""
    cfg = synth.CONFIGS["llada8b-layer"].with_(W=2)
    assert run_chained(P, cfg, steps=4, score_only_from=2) == 0


def test_dream_layer_chained(P):
    cfg = synth.CONFIGS["dream7b-layer"]
    assert run_chained(P, cfg, steps=3) == 0


def test_full_size_llada_batch_sampled(P):
    """512 windows (32 layers x 16 sequences) in one launch per call, as the
    benchmark runs them; windows 0, 301 and 511 checked against the oracle."""
    cfg = synth.CONFIGS["llada8b-batch"]
    assert run_chained(P, cfg, steps=3, windows=[0, 301, 511]) == 0


@pytest.mark.timeout(900)
def test_full_size_long_window_sampled(P):
    """128 windows of 8192 tokens, K = 256, all eight Lloyd iterations per
    step, in one launch per call as the benchmark runs them; windows 5 and 77
    checked against the oracle over window formation and one drift step (the
    oracle takes about a minute per window-step at this size, one host thread
    per window)."""
    cfg = synth.CONFIGS["llada8b-long"]
    assert run_chained(P, cfg, steps=2, windows=[5, 77]) == 0


def test_step_is_deterministic(P):
    """The same inputs twice give bit-identical outputs (no float atomics)."""
    from drift_aware_kv_amd.pipeline import DriftPath, StepSpec
    cfg = synth.CONFIGS["llada8b-layer"].with_(W=4)
    spec = StepSpec(W=4, N=cfg.N, d=cfg.d, Hq=cfg.Hq, Hkv=cfg.Hkv, dh=cfg.dh, Nb=cfg.Nb, K=cfg.K,
                    k=cfg.k, iters=cfg.iters, bf16=True, softmax_scale=cfg.softmax_scale)
    data = synth.generate(cfg)
    ins = [dev(data[k]) for k in ("H", "Kr", "V", "Q")]
    outs = []
    for rep in range(2):
        p = DriftPath(spec)
        p.step(*ins)
        ins[0][:, :60].mul_(-1)  # some drift for step 1
        p.step(*ins)
        ins[0][:, :60].mul_(-1)
        torch.cuda.synchronize()
        outs.append([host(x).copy() for x in (p.C, p.assign, p.Ck, p.codes, p.logp[1], p.score,
                                              p.idx, p.pos, p.H_hat)])
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_windows_are_independent_of_the_batch(P):
    """A window's step outputs are bit-identical whether it runs alone or in a
    batch with others: no kernel reads another window's data, and no result
    depends on how many windows a launch covers."""
    from drift_aware_kv_amd.pipeline import DriftPath, StepSpec
    cfg = synth.CONFIGS["llada8b-layer"].with_(W=3)

    def spec_for(W):
        return StepSpec(W=W, N=cfg.N, d=cfg.d, Hq=cfg.Hq, Hkv=cfg.Hkv, dh=cfg.dh, Nb=cfg.Nb, K=cfg.K,
                        k=cfg.k, iters=cfg.iters, bf16=True, softmax_scale=cfg.softmax_scale,
                        block_start=cfg.block_start)

    data = synth.generate(cfg)
    steps = []
    for t in range(3):
        if t:
            synth.apply_drift(cfg, data, t)
        steps.append({k: data[k].copy() for k in ("H", "Kr", "V", "Q")} | {"conf": synth.confidences(cfg, t)})
    names = ("C", "assign", "counts", "row_norm", "Ck", "codes", "bscale", "rscale", "D_i", "score", "idx",
             "pos", "count", "H_hat", "K_out", "V_out", "commit_block", "commit_suffix", "suffix_flag")
    batch = DriftPath(spec_for(3))
    for st in steps:
        batch.step(*[dev(st[k]) for k in ("H", "Kr", "V", "Q", "conf")])
    torch.cuda.synchronize()
    for w in range(3):
        say("window", w, "alone")
        alone = DriftPath(spec_for(1))
        for st in steps:
            alone.step(*[dev(st[k][w:w + 1]) for k in ("H", "Kr", "V", "Q", "conf")])
        torch.cuda.synchronize()
        for name in names:
            a = host(getattr(batch, name))[w:w + 1]
            b = host(getattr(alone, name))
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (w, name)


@pytest.mark.parametrize("name,W,steps", [("llada8b-batch", 48, 4), ("llada8b-long", 6, 3)])
def test_fixed_point_exit_equals_every_pass_over_steps(P, name, W, steps):
    """Whole steps with the default K-Means (a window's Lloyd passes stop once
    one moves no row) and with every pass run in full, on the same device
    inputs (the benchmark's generator, fewer windows): every output of every
    step bit-identical."""
    from drift_aware_kv_amd.pipeline import DriftPath, StepSpec
    from synth.device import DeviceWorkload
    cfg = synth.CONFIGS[name].with_(W=W)
    wl = DeviceWorkload(cfg, steps)
    paths = []
    for flags in (P.PS_KMEANS_DEFAULT, P.PS_KMEANS_ALL_PASSES):
        spec = StepSpec(W=W, N=cfg.N, d=cfg.d, Hq=cfg.Hq, Hkv=cfg.Hkv, dh=cfg.dh, Nb=cfg.Nb, K=cfg.K,
                        k=cfg.k, iters=cfg.iters, bf16=True, softmax_scale=cfg.softmax_scale,
                        block_start=cfg.block_start, kmeans_flags=flags)
        paths.append(DriftPath(spec))
    names = ("C", "assign", "counts", "row_norm", "Ck", "codes", "bscale", "rscale", "D_i", "score", "idx",
             "pos", "count", "H_hat", "K_out", "V_out", "commit_block", "commit_suffix", "suffix_flag")
    for t in range(steps):
        say(f"  {name} step {t}")
        for p in paths:
            p.step(*wl.inputs(t))
        torch.cuda.synchronize()
        for key in names:
            a, b = host(getattr(paths[0], key)), host(getattr(paths[1], key))
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (t, key)
