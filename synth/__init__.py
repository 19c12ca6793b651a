"""Seeded synthetic workloads for the Polestar-Cache drift-detection path.

This module only *generates inputs*: window hidden states, key/value rows and
decode-block queries shaped like single layers (or whole-model batches) of
LLaDA-8B and Dream-7B, plus the per-step drift that the next denoising step
sees.  It holds none of the method's arithmetic and is shared, unchanged, by
the CPU oracle side and the GPU side of every check and of the benchmark.

The real hidden states of those models on GSM8K / MATH / HumanEval / MBPP /
ParallelBench are not available; these synthetic tensors stand in for them
with the layer shapes of the workloads below.

bf16 tensors are numpy ``uint16`` bit patterns; fp32 tensors are ``float32``.
"""
import ctypes
import os
from dataclasses import dataclass, replace

import numpy as np

from . import build as _build

BASE_SEED = 20260717

# stream ids of the counter-based generator
S_H, S_KR, S_V, S_Q, S_DIR, S_LAB = 1, 2, 3, 4, 5, 6


def _conf_stream(t):
    """Per-position token confidences at denoising step t."""
    return 3000 + t


def _drift_pick_stream(t):
    return 100 + t


def _drift_noise_stream(t, tensor):
    return 1000 + 10 * t + tensor


@dataclass(frozen=True)
class Config:
    name: str
    W: int          # windows = sequences x layers
    N: int          # window tokens (prefix + decode block + suffix)
    d: int          # hidden size
    Hq: int
    Hkv: int
    dh: int
    Nb: int         # decode-block rows (queries)
    K: int          # clusters
    k: int          # top-k clusters refreshed
    iters: int      # Lloyd iterations per step
    steps: int      # denoising steps of the recipe
    dtype: str      # "f32" or "bf16"
    init0: str      # seeding at window formation: "farthest" or "strided"
    drift: str      # "gauss", "rotate" or "student"
    drift_frac: float
    drift_mag: float
    planted: bool = False

    @property
    def block_start(self) -> int:
        return (self.N - self.Nb) // 2

    @property
    def drift_rows(self) -> int:
        return int(round(self.drift_frac * self.N))

    @property
    def bf16(self) -> bool:
        return self.dtype == "bf16"

    @property
    def softmax_scale(self) -> float:
        return float(np.float32(1.0 / np.sqrt(self.dh)))

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


CONFIGS = {
    # tiny case: 8 planted unit directions + N(0, 0.05^2) noise, d = 64 fp32,
    # 1 head whose queries are the block's hidden rows, Kr = V = H.
    "tiny-planted": Config("tiny-planted-N256-d64-K8", W=1, N=256, d=64, Hq=1, Hkv=1, dh=64, Nb=16, K=8,
                 k=2, iters=10, steps=2, dtype="f32", init0="farthest", drift="gauss",
                 drift_frac=0.10, drift_mag=0.3, planted=True),
    # LLaDA-8B-shaped single layer
    "llada8b-layer": Config("llada8b-layer-N1024-K64", W=1, N=1024, d=4096, Hq=32, Hkv=32, dh=128, Nb=32,
                 K=64, k=4, iters=8, steps=20, dtype="bf16", init0="strided", drift="gauss",
                 drift_frac=0.05, drift_mag=0.3),
    # Dream-7B-shaped single layer (GQA 28/4)
    "dream7b-layer": Config("dream7b-layer-N2048-K128", W=1, N=2048, d=3584, Hq=28, Hkv=4, dh=128, Nb=32,
                 K=128, k=8, iters=8, steps=20, dtype="bf16", init0="strided", drift="rotate",
                 drift_frac=0.10, drift_mag=0.2),
    # LLaDA-8B, all 32 layers x 16 sequences
    "llada8b-batch": Config("llada8b-32layers-16seq-N1024-K64", W=512, N=1024, d=4096, Hq=32, Hkv=32,
                 dh=128, Nb=32, K=64, k=4, iters=8, steps=20, dtype="bf16", init0="strided",
                 drift="gauss", drift_frac=0.05, drift_mag=0.3),
    # long window stress: LLaDA-8B, 32 layers x 4 sequences, N = 8192
    "llada8b-long": Config("llada8b-32layers-4seq-N8192-K256", W=128, N=8192, d=4096, Hq=32, Hkv=32,
                 dh=128, Nb=32, K=256, k=16, iters=8, steps=64, dtype="bf16", init0="strided",
                 drift="student", drift_frac=0.10, drift_mag=0.3),
}


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        u64, i32, i64, dbl, P = (ctypes.c_uint64, ctypes.c_int, ctypes.c_int64, ctypes.c_double,
                                 ctypes.c_void_p)
        L.synth_normal.argtypes = [u64, u64, u64, i64, dbl, i32, P]
        L.synth_uniform.argtypes = [u64, u64, u64, i64, dbl, dbl, P]
        L.synth_planted.argtypes = [u64, i32, i32, i32, dbl, P, P]
        L.synth_pick_rows.argtypes = [u64, u64, i32, i32, i32, P]
        L.synth_add_noise_rows.argtypes = [u64, u64, i32, i32, i32, i32, i32, P, dbl, i32, i32, P]
        L.synth_rotate_rows.argtypes = [u64, u64, i32, i32, i32, i32, i32, P, dbl, i32, P]
        for f in ("synth_normal", "synth_uniform", "synth_planted", "synth_pick_rows", "synth_add_noise_rows",
                  "synth_rotate_rows"):
            getattr(L, f).restype = None
        _lib = L
    return _lib


def _ptr(a):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def normal(shape, seed, stream, offset=0, scale=1.0, bf16=True):
    """scale * N(0,1), element i of the array = element offset+i of the stream."""
    out = np.empty(shape, np.uint16 if bf16 else np.float32)
    lib().synth_normal(seed, stream, offset, out.size, scale, 1 if bf16 else 0, _ptr(out))
    return out


def uniform(shape, seed, stream, offset=0, lo=0.0, hi=1.0):
    """fp32 lo + (hi - lo) * U(0,1); element i = element offset+i of the stream."""
    out = np.empty(shape, np.float32)
    lib().synth_uniform(seed, stream, offset, out.size, lo, hi, _ptr(out))
    return out


def confidences(cfg: "Config", t: int, w0: int = 0, Wc: int = None, seed: int = BASE_SEED):
    """Stand-in for the model's per-position confidence (the probability of
    its predicted token) at step t: U(0,1), [Wc][N] fp32."""
    Wc = cfg.W - w0 if Wc is None else Wc
    return uniform((Wc, cfg.N), seed, _conf_stream(t), offset=w0 * cfg.N)


def planted(N, d, M, noise, seed=BASE_SEED):
    out = np.empty((N, d), np.float32)
    lab = np.empty((N,), np.int32)
    lib().synth_planted(seed, N, d, M, noise, _ptr(out), _ptr(lab))
    return out, lab


def pick_rows(seed, t, w, N, count):
    rows = np.empty((count,), np.int32)
    lib().synth_pick_rows(seed, _drift_pick_stream(t), w, N, count, _ptr(rows))
    return rows


def generate(cfg: Config, w0: int = 0, Wc: int = None, seed: int = BASE_SEED):
    """Step-0 inputs of windows [w0, w0+Wc): dict of H [Wc][N][d],
    Kr and V [Wc][N][Hkv][dh], Q [Wc][Nb][Hq][dh] (and labels for the
    planted case)."""
    Wc = cfg.W - w0 if Wc is None else Wc
    N, d = cfg.N, cfg.d
    if cfg.planted:
        assert cfg.Hq == 1 and cfg.Hkv == 1 and cfg.dh == d
        Hs, labs = [], []
        for w in range(w0, w0 + Wc):
            h, lab = planted(N, d, cfg.K, 0.05, seed=seed + w)
            Hs.append(h)
            labs.append(lab)
        H = np.stack(Hs)
        out = dict(H=H, labels=np.stack(labs))
        _planted_views(cfg, out)
        return out
    bf = cfg.bf16
    KV = cfg.Hkv * cfg.dh
    H = normal((Wc, N, d), seed, S_H, offset=w0 * N * d, bf16=bf)
    Kr = normal((Wc, N, cfg.Hkv, cfg.dh), seed, S_KR, offset=w0 * N * KV, bf16=bf)
    V = normal((Wc, N, cfg.Hkv, cfg.dh), seed, S_V, offset=w0 * N * KV, bf16=bf)
    Q = normal((Wc, cfg.Nb, cfg.Hq, cfg.dh), seed, S_Q, offset=w0 * cfg.Nb * cfg.Hq * cfg.dh,
               bf16=bf)
    return dict(H=H, Kr=Kr, V=V, Q=Q)


def _planted_views(cfg, data):
    """Planted case: the key and value rows are the hidden rows, and the single
    query head reads the decode block's hidden rows."""
    H = data["H"]
    Wc = H.shape[0]
    data["Kr"] = H.reshape(Wc, cfg.N, 1, cfg.d).copy()
    data["V"] = H.reshape(Wc, cfg.N, 1, cfg.d).copy()
    b0 = cfg.block_start
    data["Q"] = H[:, b0:b0 + cfg.Nb, :].reshape(Wc, cfg.Nb, 1, cfg.d).copy()


def apply_drift(cfg: Config, data: dict, t: int, w0: int = 0, seed: int = BASE_SEED):
    """Move the inputs from step t-1 to step t in place (t >= 1) and return the
    perturbed rows, [Wc][drift_rows] int32 ascending per window."""
    assert t >= 1
    H = data["H"]
    Wc, N = H.shape[0], cfg.N
    n = cfg.drift_rows
    rows = np.stack([pick_rows(seed, t, w0 + w, N, n) for w in range(Wc)]).astype(np.int32)
    rows = np.ascontiguousarray(rows)
    L = lib()
    bf = 1 if cfg.bf16 else 0
    kind = {"gauss": 0, "student": 1}.get(cfg.drift)

    def perturb(arr, tensor, Nrows, rws, w_first, Wn):
        length = int(np.prod(arr.shape[2:]))
        nr = rws.shape[1]
        if nr == 0:
            return
        stream = _drift_noise_stream(t, tensor)
        if cfg.drift == "rotate":
            L.synth_rotate_rows(seed, stream, w_first, Wn, Nrows, length, nr, _ptr(rws),
                                cfg.drift_mag, bf, _ptr(arr))
        else:
            L.synth_add_noise_rows(seed, stream, w_first, Wn, Nrows, length, nr, _ptr(rws),
                                   cfg.drift_mag, kind, bf, _ptr(arr))

    perturb(H, 1, N, rows, w0, Wc)
    if cfg.planted:
        _planted_views(cfg, data)
        return rows
    perturb(data["Kr"], 2, N, rows, w0, Wc)
    perturb(data["V"], 3, N, rows, w0, Wc)
    b0 = cfg.block_start
    Q = data["Q"]
    for w in range(Wc):
        qr = rows[w][(rows[w] >= b0) & (rows[w] < b0 + cfg.Nb)] - b0
        if qr.size == 0:
            continue
        qr = np.ascontiguousarray(qr.reshape(1, -1).astype(np.int32))
        Qw = Q[w:w + 1]
        perturb(Qw, 4, cfg.Nb, qr, w0 + w, 1)
    return rows


def window_at_step(cfg: Config, w: int, t: int, seed: int = BASE_SEED):
    """Inputs of the single window w at step t (step 0 plus drifts 1..t),
    generated independently of the other windows."""
    data = generate(cfg, w0=w, Wc=1, seed=seed)
    for s in range(1, t + 1):
        apply_drift(cfg, data, s, w0=w, seed=seed)
    return data
