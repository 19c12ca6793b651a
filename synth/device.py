"""Device-side seeded workloads for the benchmark.

Same recipe as the host generator in this package (N(0,1) hidden states, key
and value rows and queries in bf16, U(0,1) per-position confidences drawn
afresh at every step; per-step drift on a seeded random subset
of round(frac * N) rows per window: Gaussian noise, Student-t (nu = 3) noise,
or a rotation by theta inside the plane of the row and a random orthogonal
direction), drawn with torch's generator on the GPU so that multi-GiB batches
never cross PCIe.  Holds none of the method's arithmetic.  Values are not
bit-identical to the host generator's (a different random stream); the parity
tests use the host generator.
"""
import torch

from . import BASE_SEED, Config


class DeviceWorkload:
    """Snapshots of the inputs at successive denoising steps, resident on the
    device: snapshot 0 is the window formation, snapshot t = snapshot t-1 plus
    the drift of step t."""

    def __init__(self, cfg: Config, n_snapshots: int, seed: int = BASE_SEED, device="cuda"):
        self.cfg = cfg
        self.dev = torch.device(device)
        self.g = torch.Generator(device=self.dev).manual_seed(seed)
        et = torch.bfloat16 if cfg.bf16 else torch.float32
        W, N = cfg.W, cfg.N
        base = dict(
            H=self._randn((W, N, cfg.d)).to(et),
            Kr=self._randn((W, N, cfg.Hkv, cfg.dh)).to(et),
            V=self._randn((W, N, cfg.Hkv, cfg.dh)).to(et),
            Q=self._randn((W, cfg.Nb, cfg.Hq, cfg.dh)).to(et),
            conf=self._rand((W, N)),
        )
        self.snaps = [base]
        for t in range(1, n_snapshots):
            nxt = {k: v.clone() for k, v in self.snaps[-1].items()}
            self._drift(nxt)
            self.snaps.append(nxt)

    def _rand(self, shape):
        return torch.rand(shape, generator=self.g, device=self.dev, dtype=torch.float32)

    def _randn(self, shape):
        return torch.randn(shape, generator=self.g, device=self.dev, dtype=torch.float32)

    def _drift(self, s):
        cfg = self.cfg
        W, N, n = cfg.W, cfg.N, cfg.drift_rows
        rows = torch.rand((W, N), generator=self.g, device=self.dev).argsort(dim=1)[:, :n]
        widx = torch.arange(W, device=self.dev)[:, None].expand(W, n)
        for key in ("H", "Kr", "V"):
            x = s[key].view(W, N, -1)
            sel = x[widx, rows].float()
            x[widx, rows] = self._move(sel).to(x.dtype)
        b0 = cfg.block_start
        inb = (rows >= b0) & (rows < b0 + cfg.Nb)
        if inb.any():
            q = s["Q"].view(W, cfg.Nb, -1)
            wq, rq = widx[inb], rows[inb] - b0
            q[wq, rq] = self._move(q[wq, rq].float()).to(q.dtype)
        s["conf"] = self._rand((W, N))      # the model's confidences change every step

    def _move(self, x):
        cfg = self.cfg
        if cfg.drift == "gauss":
            return x + cfg.drift_mag * self._randn(x.shape)
        if cfg.drift == "student":
            z = self._randn(x.shape)
            chi = sum(self._randn(x.shape) ** 2 for _ in range(3))
            return x + cfg.drift_mag * z / torch.sqrt(chi / 3.0)
        # rotation by theta towards a random direction orthogonal to the row
        g = self._randn(x.shape)
        hn = x.norm(dim=-1, keepdim=True).clamp_min(1e-30)
        u = g - (g * x).sum(-1, keepdim=True) / hn ** 2 * x
        u = u / u.norm(dim=-1, keepdim=True).clamp_min(1e-30)
        th = torch.tensor(cfg.drift_mag)
        return torch.cos(th) * x + torch.sin(th) * hn * u

    def inputs(self, step: int):
        """Snapshot used at `step`: the sequence runs through the snapshots once,
        then cycles over snapshots 1.. (the wrap is a larger, still valid drift)."""
        S = len(self.snaps)
        i = step if step < S else 1 + (step - 1) % (S - 1) if S > 1 else 0
        s = self.snaps[i]
        return s["H"], s["Kr"], s["V"], s["Q"], s["conf"]

    @staticmethod
    def snapshot_bytes(cfg: Config) -> int:
        e = 2 if cfg.bf16 else 4
        return (e * cfg.W * (cfg.N * cfg.d + 2 * cfg.N * cfg.Hkv * cfg.dh + cfg.Nb * cfg.Hq * cfg.dh)
                + 4 * cfg.W * cfg.N)
