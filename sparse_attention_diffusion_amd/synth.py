"""Seeded synthetic Q/K/V for the attention workloads in ``configs``.

This module is the one piece shared by the GPU tests, the oracle tests and the
benchmark.  It holds no attention arithmetic: it only draws inputs.

Recipe (stated once, used everywhere):

* Tokens: ``n_text`` text tokens first, then the latent grid in row-major order
  ((y, x) for images, (t, y, x) for video).  Grid coordinates are normalised to
  [0, 1) per axis (``t/T``, ``y/Hg``, ``x/Wg``).
* Step 0, latent tokens: for each tensor X in (Q, K, V), each (b, h) and each
  channel c < d, a smooth field made of 4 sinusoids of the coordinates,
  ``sum_i sin(2*pi*<kappa_i, u> + phi_i)`` with integer wave vectors kappa_i drawn
  uniformly from [-3, 3]^dim without the zero vector and phases phi_i uniform in
  [0, 2*pi); each term has amplitude 1.  Gaussian noise of standard deviation
  0.5 is added.
* Step 0, text tokens: standard normal features.
* Step s -> s+1 (denoising drift): X <- 0.98 * X + 0.2 * noise on every token.
* Channels d..d_pad-1 are zero at every step.
* Values are produced in float32 and then stored as the workload's dtype
  (bf16 rounds to nearest even); every consumer sees the stored values.

Draw order from one ``torch.Generator`` seeded with ``seed``: kappa and phi for
Q, K, V; step-0 noise for Q, K, V; then per drift step noise for Q, K, V.
A CPU generator and a GPU generator give different (each reproducible) streams.
"""
import math

import torch

from .configs import check

NOISE0 = 0.5
DRIFT_DECAY = 0.98
DRIFT_NOISE = 0.2
N_TERMS = 4
KAPPA_MAX = 3


def coords(cfg, device="cpu"):
    """Normalised grid coordinates of the latent tokens, [n_grid, dim] float32."""
    g = cfg["grid"]
    sizes = g[1:]
    axes = [torch.arange(s, device=device, dtype=torch.float32) / s for s in sizes]
    mesh = torch.meshgrid(*axes, indexing="ij")
    return torch.stack([m.reshape(-1) for m in mesh], dim=1)


def _nonzero_lattice(dim, device):
    side = 2 * KAPPA_MAX + 1
    pts = torch.cartesian_prod(*[torch.arange(-KAPPA_MAX, KAPPA_MAX + 1, device=device)] * dim)
    if dim == 1:
        pts = pts.reshape(-1, 1)
    keep = (pts != 0).any(dim=1)
    out = pts[keep].to(torch.float32)
    assert out.shape[0] == side ** dim - 1
    return out


class StepInputs:
    """Iterates the per-step (q, k, v) of one layer of a workload."""

    def __init__(self, cfg, seed=0, device="cpu", heads=None):
        self.cfg = check(dict(cfg))
        self.device = torch.device(device)
        self.gen = torch.Generator(device=self.device)
        self.gen.manual_seed(int(seed))
        B, H, N, d, D = (self.cfg[x] for x in ("B", "H", "N", "d", "d_pad"))
        self.shape = (B, H, N, D)
        self.d = d
        self.step = -1
        self._x = None

    def _field(self, lattice, u):
        B, H, N, D = self.shape
        d = self.d
        dim = u.shape[1]
        idx = torch.randint(0, lattice.shape[0], (B, H, d, N_TERMS), generator=self.gen, device=self.device)
        phi = torch.rand((B, H, d, N_TERMS), generator=self.gen, device=self.device) * (2 * math.pi)
        kappa = lattice[idx]  # [B,H,d,T,dim]
        out = torch.empty((B, H, u.shape[0], d), dtype=torch.float32, device=self.device)
        for b in range(B):
            for h in range(H):
                ang = (2 * math.pi) * (u @ kappa[b, h].reshape(d * N_TERMS, dim).T)  # [n, d*T]
                ang = ang + phi[b, h].reshape(1, d * N_TERMS)
                out[b, h] = torch.sin(ang).reshape(-1, d, N_TERMS).sum(dim=2)
        return out

    def _initial(self):
        B, H, N, D = self.shape
        d = self.d
        nt = self.cfg["n_text"]
        u = coords(self.cfg, self.device)
        lattice = _nonzero_lattice(u.shape[1], self.device)
        fields = [self._field(lattice, u) for _ in range(3)]
        xs = []
        for f in fields:
            eps = torch.randn((B, H, N, d), generator=self.gen, device=self.device)
            x = torch.zeros((B, H, N, D), dtype=torch.float32, device=self.device)
            x[:, :, :nt, :d] = eps[:, :, :nt]
            x[:, :, nt:, :d] = f + NOISE0 * eps[:, :, nt:]
            xs.append(x)
        return xs

    def _drift(self):
        B, H, N, D = self.shape
        d = self.d
        for x in self._x:
            eps = torch.randn((B, H, N, d), generator=self.gen, device=self.device)
            x[..., :d].mul_(DRIFT_DECAY).add_(eps, alpha=DRIFT_NOISE)

    def next(self):
        """Advance one denoising step; returns fp32 (q, k, v) [B,H,N,d_pad]."""
        if self._x is None:
            self._x = self._initial()
        else:
            self._drift()
        self.step += 1
        return tuple(self._x)

    def next_stored(self):
        """Advance one step; returns (q, k, v) in the workload's storage dtype."""
        q, k, v = self.next()
        return tuple(store(t, self.cfg["dtype"]) for t in (q, k, v))


def store(t, dtype):
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t.clone()
    raise ValueError(dtype)


def steps(cfg, n_steps, seed=0, device="cpu"):
    """List of the first ``n_steps`` stored (q, k, v) triples."""
    it = StepInputs(cfg, seed=seed, device=device)
    return [it.next_stored() for _ in range(n_steps)]


def random_qkv(B, H, N, d, d_pad, seed=0, scale=1.0, dtype="f32", device="cpu"):
    """Plain Gaussian (q, k, v) for edge-case tests, zero in the padded channels."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    out = []
    for _ in range(3):
        x = torch.zeros((B, H, N, d_pad), dtype=torch.float32, device=device)
        x[..., :d] = torch.randn((B, H, N, d), generator=g, device=device) * scale
        out.append(store(x, dtype))
    return tuple(out)
