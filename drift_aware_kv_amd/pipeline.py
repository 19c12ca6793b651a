"""One denoising step of the drift-detection path over W windows.

``DriftPath`` owns the cross-step state that the C ABI leaves to the caller
(centres C, centroid keys Ck, the previous step's log-probabilities) plus the
output buffers, all allocated once with torch on the device, and issues the
library calls in the order of one step:

  kmeans_fit -> residual_nvfp4 -> proxy_attn (+ drift) -> topk -> refresh_gather
  [-> commit_block -> commit_suffix, when per-position confidences are given]

Step 0 (window formation) seeds the clusters and stores the first proxy
distribution; there is no previous distribution, so no drift, selection or
gather happens (Polestar technical summary 2.A, schedule: a refresh follows
formation).  Later steps warm-start K-Means from the previous centres, so
cluster k at step t continues cluster k at step t-1 and the KL between the two
proxy distributions is defined.

With ``cluster_score="cosine"`` the clusters are ranked instead by how far
their centres moved during the step's K-Means (cosine dissimilarity, the
measure the pages' drift-measurement item compares KL against); the proxy
attention and its per-token drift still run for the commit rules.

Polestar-Commit (technical summary 2.B) runs on the drift of every step after
formation: the current-block rule keeps a per-row drift history (reset when a
window is formed), the suffix rule reads this step's top-k clusters.  The
pages give no values for alpha and tau_s; the defaults here are placeholders
that a caller sets.
"""
from dataclasses import dataclass

import torch

from . import (PS_BF16, PS_F32, PS_INIT_FARTHEST, PS_INIT_GIVEN, PS_INIT_STRIDED,
               PS_SCORE_KL_SHARE, Shape, ps_commit_block, ps_commit_suffix, ps_drift_cosine,
               ps_kmeans_fit, ps_kmeans_fit_nvfp4, ps_proxy_attn, ps_refresh_gather, ps_residual_nvfp4,
               ps_topk_clusters, workspace)


@dataclass
class _Store:
    codes: torch.Tensor
    bscale: torch.Tensor
    rscale: torch.Tensor


@dataclass
class StepSpec:
    W: int
    N: int
    d: int
    Hq: int
    Hkv: int
    dh: int
    Nb: int
    K: int
    k: int
    iters: int
    bf16: bool
    init0: str = "strided"
    softmax_scale: float = None
    cap: int = None
    score_kind: int = PS_SCORE_KL_SHARE
    gather_rows: bool = True
    kmeans_flags: int = 0
    block_start: int = None      # default: the block centred in the window
    alpha: float = 0.1
    tau_s: float = 0.9
    cluster_score: str = "kl"    # "kl" (drift share) or "cosine" (centre movement)
    residual_store: str = "device"  # "device" (HBM) or "host" (pinned host memory)
    fused_coding: bool = True    # K-Means and the residual coding in one call (the same results)

    @property
    def shape(self) -> Shape:
        return Shape(self.W, self.N, self.d, self.Hq, self.Hkv, self.dh, self.Nb, self.K)


class DriftPath:
    def __init__(self, spec: StepSpec, device="cuda"):
        self.spec = spec
        self.device = torch.device(device)
        s = spec.shape
        self.shape = s
        self.dtype = PS_BF16 if spec.bf16 else PS_F32
        et = torch.bfloat16 if spec.bf16 else torch.float32
        self.cap = spec.N if spec.cap is None else spec.cap
        self.scale = spec.softmax_scale if spec.softmax_scale is not None else spec.dh ** -0.5
        dev = self.device
        f32, i32 = torch.float32, torch.int32
        self.C = torch.zeros(s.W, s.K, s.d, dtype=f32, device=dev)
        self.Ck = torch.zeros(s.W, s.K, s.Hkv, s.dh, dtype=et, device=dev)
        self.assign = torch.zeros(s.W, s.N, dtype=i32, device=dev)
        self.counts = torch.zeros(s.W, s.K, dtype=i32, device=dev)
        self.row_norm = torch.zeros(s.W, s.N, dtype=f32, device=dev)
        self.objective = torch.zeros(s.W, dtype=torch.float64, device=dev)
        self.ws = workspace(s, self.dtype, dev)
        self.codes = torch.zeros(s.W, s.N, s.d // 2, dtype=torch.uint8, device=dev)
        self.bscale = torch.zeros(s.W, s.N, s.d // 16, dtype=torch.uint8, device=dev)
        self.rscale = torch.zeros(s.W, s.N, dtype=f32, device=dev)
        if spec.residual_store not in ("device", "host"):
            raise ValueError(f"residual_store must be 'device' or 'host', not {spec.residual_store!r}")
        self.store = None
        if spec.residual_store == "host":
            # the pages' CPU offload: the quantised residual store lives in
            # pinned host memory, written by a copy engine on its own stream
            # while proxy attention and top-k run, and the gather fetches only
            # the selected rows from it
            self.store = dict(codes=torch.zeros(self.codes.shape, dtype=torch.uint8, pin_memory=True),
                              bscale=torch.zeros(self.bscale.shape, dtype=torch.uint8, pin_memory=True),
                              rscale=torch.zeros(self.rscale.shape, dtype=f32, pin_memory=True))
            self.copy_stream = torch.cuda.Stream(device=dev)
            self.coded, self.stored = torch.cuda.Event(), torch.cuda.Event()
        self.logp = [torch.zeros(s.W, s.Hq, s.Nb, s.K, dtype=f32, device=dev) for _ in range(2)]
        self.D_hi = torch.zeros(s.W, s.Hq, s.Nb, dtype=f32, device=dev)
        self.D_i = torch.zeros(s.W, s.Nb, dtype=f32, device=dev)
        self.score = torch.zeros(s.W, s.K, dtype=f32, device=dev)
        if spec.cluster_score not in ("kl", "cosine"):
            raise ValueError(f"cluster_score must be 'kl' or 'cosine', not {spec.cluster_score!r}")
        self.C_prev = self.score_cos = None
        if spec.cluster_score == "cosine":
            self.C_prev = torch.zeros_like(self.C)
            self.score_cos = torch.zeros(s.W, s.K, dtype=f32, device=dev)
        self.idx = torch.zeros(s.W, spec.k, dtype=i32, device=dev)
        self.val = torch.zeros(s.W, spec.k, dtype=f32, device=dev)
        self.pos = torch.full((s.W, max(self.cap, 1)), -1, dtype=i32, device=dev)
        self.count = torch.zeros(s.W, dtype=i32, device=dev)
        if spec.gather_rows and self.cap > 0:
            self.H_hat = torch.zeros(s.W, self.cap, s.d, dtype=et, device=dev)
            self.K_out = torch.zeros(s.W, self.cap, s.Hkv, s.dh, dtype=et, device=dev)
            self.V_out = torch.zeros(s.W, self.cap, s.Hkv, s.dh, dtype=et, device=dev)
        else:
            self.H_hat = self.K_out = self.V_out = None
        self.block_start = (s.N - s.Nb) // 2 if spec.block_start is None else spec.block_start
        self.hist_sum = torch.zeros(s.W, s.Nb, dtype=torch.float64, device=dev)
        self.hist_n = torch.zeros(s.W, dtype=i32, device=dev)
        self.commit_block = torch.zeros(s.W, s.Nb, dtype=torch.uint8, device=dev)
        self.delta = torch.zeros(s.W, s.Nb, dtype=f32, device=dev)
        self.suffix_flag = torch.zeros(s.W, dtype=torch.uint8, device=dev)
        self.commit_suffix = torch.zeros(s.W, s.N, dtype=torch.uint8, device=dev)
        self.t = 0
        self._graphs = {}

    @property
    def logp_cur(self):
        return self.logp[self.t & 1]

    @property
    def logp_prev(self):
        return self.logp[(self.t - 1) & 1]

    def step(self, H, Kr, V, Q, conf=None, stream=None, recluster=True):
        """Run one step on device tensors H [W][N][d], Kr/V [W][N][Hkv][dh],
        Q [W][Nb][Hq][dh] and, optionally, the per-position confidences
        conf [W][N] f32 that the commit rules read; returns t of the step just
        run.  recluster=False keeps the clusters, centroid keys and residual
        codes of the last clustered step and runs only the scoring half
        (proxy attention and drift, top-k, gather, commit rules): the reading
        in which clustering happens at window formation only."""
        sp, s, dt = self.spec, self.shape, self.dtype
        first = self.t == 0
        if not recluster and (first or self.score_cos is not None):
            raise ValueError("recluster=False needs a formed window and the KL cluster score")
        init = {"strided": PS_INIT_STRIDED, "farthest": PS_INIT_FARTHEST}[sp.init0] if first \
            else PS_INIT_GIVEN
        cosine = self.score_cos is not None and not first
        if cosine:
            with torch.cuda.stream(stream if stream is not None else torch.cuda.current_stream()):
                self.C_prev.copy_(self.C)
        if recluster and sp.fused_coding:
            ps_kmeans_fit_nvfp4(s, dt, H, Kr, init, sp.iters, self.C, self.assign, self.counts, self.row_norm,
                                self.codes, self.bscale, self.rscale, self.Ck, self.objective, self.ws, stream,
                                flags=sp.kmeans_flags)
        elif recluster:
            ps_kmeans_fit(s, dt, H, Kr, init, sp.iters, self.C, self.assign, self.counts, self.row_norm,
                          self.Ck, self.objective, self.ws, stream, flags=sp.kmeans_flags)
            ps_residual_nvfp4(s, dt, H, self.row_norm, self.C, self.assign, self.codes, self.bscale,
                              self.rscale, self.ws, stream)
        main = stream if stream is not None else torch.cuda.current_stream()
        if self.store is not None and not first:     # formation gathers nothing
            self.coded.record(main)
            with torch.cuda.stream(self.copy_stream):
                self.copy_stream.wait_event(self.coded)
                for key in ("codes", "bscale", "rscale"):
                    self.store[key].copy_(getattr(self, key), non_blocking=True)
                self.stored.record(self.copy_stream)
        ps_proxy_attn(s, dt, Q, self.Ck, self.scale, self.logp_cur, None if first else self.logp_prev,
                      sp.score_kind, self.D_hi, self.D_i, self.score, stream)
        if not first:
            score = self.score
            if cosine:
                ps_drift_cosine(s, self.C, self.C_prev, self.score_cos, stream)
                score = self.score_cos
            ps_topk_clusters(s, score, sp.k, self.idx, self.val, stream)
            gather = self.K_out is not None
            src = self
            if self.store is not None:
                main.wait_event(self.stored)
                src = _Store(**self.store)
            ps_refresh_gather(s, dt, self.assign, self.idx, sp.k, self.cap,
                              self.pos if self.cap > 0 else None, self.count, src.codes,
                              src.bscale, src.rscale, self.C, self.row_norm, self.H_hat,
                              Kr if gather else None, V if gather else None, self.K_out,
                              self.V_out, stream)
            if conf is not None:
                ps_commit_block(s, self.D_i, conf, self.block_start, sp.alpha, sp.tau_s,
                                self.hist_sum, self.hist_n, self.commit_block, self.delta, stream)
                ps_commit_suffix(s, self.assign, self.idx, sp.k, self.block_start, conf, sp.tau_s,
                                 self.suffix_flag, self.commit_suffix, stream)
        t = self.t
        self.t += 1
        return t

    def step_graphed(self, H, Kr, V, Q, conf=None):
        """The same step as step(), replayed from a HIP graph.

        Steps after window formation launch the same kernels with the same
        arguments whenever the input buffers and the parity of t (which of the
        two log-probability buffers is current) repeat, so one graph per such
        key is captured on first use and replayed after that: one submission
        instead of one launch per kernel.  Formation runs eagerly.  Inputs must
        stay at their addresses; the residual store must be on the device; the
        kernel timer must be off.  Runs on the current stream."""
        if self.t == 0:
            return self.step(H, Kr, V, Q, conf)
        if self.store is not None:
            raise ValueError("step_graphed needs the residual store on the device")
        key = (H.data_ptr(), Kr.data_ptr(), V.data_ptr(), Q.data_ptr(),
               conf.data_ptr() if conf is not None else 0, self.t & 1)
        g = self._graphs.get(key)
        if g is None:
            g = torch.cuda.CUDAGraph()
            t = self.t
            with torch.cuda.graph(g):
                self.step(H, Kr, V, Q, conf)      # recorded, not run
            self.t = t
            self._graphs[key] = g
        g.replay()
        t = self.t
        self.t += 1
        return t
