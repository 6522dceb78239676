"""Seeded synthetic video-token tensors for the five block-sparse attention workloads.

This module only draws random numbers and smooths them. It holds none of the
attention method's arithmetic (no reordering, pooling, scoring or masking), so
the CPU oracle and the HIP path can both consume what it produces without
sharing any of the computation under test.

The NABLA and DynamicRad pages evaluate trained video DiTs (Wan 2.1, HunyuanVideo)
on real videos. Neither the models nor the videos are available, so these fields
stand in for the Q/K/V of one attention layer: spatially smooth, temporally
correlated and with a few exact long-range repeats, which is the structure the
content-adaptive mask is meant to exploit.

Layout of every tensor: [B, H, N, d] with N = T*Hs*Ws in the natural
(frame, row, column) order n = (t*Hs + y)*Ws + x.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

GENERATOR_VERSION = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention-layer workload: geometry, dtype, field recipe and mask parameters."""

    name: str
    B: int
    H: int
    d: int
    T: int
    Hs: int
    Ws: int
    P: int
    dtype: str  # "f32" or "bf16"
    recipe: str  # "tiny" (3D-smoothed shared field + noise) or "video" (2D-smoothed AR(1) + copies)
    sigma: float  # smoothing width in tokens
    rho: float = 0.0  # lag-1 temporal correlation (video recipe)
    copy_frac: float = 0.0  # fraction of blocks overwritten by a distant block (video recipe)
    qk_noise: float = 0.0  # std of independent noise added to Q and K before normalisation
    mode: str = "cdf"  # "cdf", "dyn" or "static"
    thr: float = 0.0
    tau: float = 0.0
    gamma: float = 0.5  # static mode: retention decay per frame of distance
    lam: float = 0.05  # static mode: long-range floor of the retention ratio
    sta: tuple = (3, 3, 3)
    seed: int = 0

    @property
    def N(self) -> int:
        return self.T * self.Hs * self.Ws

    @property
    def nb(self) -> int:
        return self.T * (self.Hs // self.P) * (self.Ws // self.P)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five benchmark workloads (geometry, dtype and mask parameters fixed by the benchmark
# definition; the field recipe is the reading written up in the design notes), plus
# 480p-static: the 480p geometry under the DynamicRad Static-Ratio mask.
WORKLOADS = {
    "tiny": Workload("tiny", B=1, H=2, d=64, T=8, Hs=16, Ws=16, P=8, dtype="f32",
                     recipe="tiny", sigma=2.0, qk_noise=0.3, mode="cdf", thr=0.8),
    "480p": Workload("480p", B=1, H=12, d=128, T=21, Hs=32, Ws=56, P=8, dtype="bf16",
                     recipe="video", sigma=3.0, rho=0.9, copy_frac=0.05, mode="cdf", thr=0.7),
    "720p": Workload("720p", B=1, H=40, d=128, T=21, Hs=48, Ws=80, P=8, dtype="bf16",
                     recipe="video", sigma=3.0, rho=0.9, copy_frac=0.05, mode="cdf", thr=0.9),
    "480p-dyn": Workload("480p-dyn", B=1, H=12, d=128, T=21, Hs=32, Ws=56, P=8, dtype="bf16",
                         recipe="video", sigma=3.0, rho=0.9, copy_frac=0.05, mode="dyn", tau=4.0),
    "480p-static": Workload("480p-static", B=1, H=12, d=128, T=21, Hs=32, Ws=56, P=8, dtype="bf16",
                            recipe="video", sigma=3.0, rho=0.9, copy_frac=0.05, mode="static", gamma=0.5,
                            lam=0.05),
    "long": Workload("long", B=1, H=12, d=128, T=105, Hs=32, Ws=56, P=8, dtype="bf16",
                     recipe="video", sigma=3.0, rho=0.95, copy_frac=0.05, mode="cdf", thr=0.9),
}


def _seed_for(seed: int, b: int, h: int, purpose: int) -> int:
    # Distinct, reproducible stream per (seed, batch, head, purpose).
    return (((seed * 1_000_003 + b) * 10_007 + h) * 101 + purpose) & 0x7FFF_FFFF_FFFF


def _gen(device, seed: int, b: int, h: int, purpose: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed_for(seed, b, h, purpose))
    return g


def _reflect_index(i: int, n: int) -> int:
    """Half-sample symmetric extension (a b c | c b a), repeated as often as needed."""
    period = 2 * n
    i = i % period
    return i if i < n else period - 1 - i


def gaussian_matrix(n: int, sigma: float, truncate: float = 4.0) -> torch.Tensor:
    """n x n matrix G with (G @ x) = 1D Gaussian smoothing of x, reflect boundaries."""
    G = torch.zeros(n, n, dtype=torch.float64)
    if sigma <= 0:
        return torch.eye(n, dtype=torch.float64)
    r = int(truncate * sigma + 0.5)
    taps = torch.tensor([math.exp(-0.5 * (k / sigma) ** 2) for k in range(-r, r + 1)], dtype=torch.float64)
    taps /= taps.sum()
    for i in range(n):
        for k in range(-r, r + 1):
            G[i, _reflect_index(i + k, n)] += taps[k + r]
    return G


def _smooth(x: torch.Tensor, axis: int, sigma: float) -> torch.Tensor:
    G = gaussian_matrix(x.shape[axis], sigma).to(device=x.device, dtype=x.dtype)
    return torch.matmul(x.movedim(axis, -1), G.T).movedim(-1, axis)


def _unit(x: torch.Tensor) -> torch.Tensor:
    s = x.double().pow(2).mean().sqrt().to(x.dtype)  # fields are zero-mean by construction
    return x / s


def _tiny_head(w: Workload, device, b: int, h: int):
    gF, gq, gk, gv = (_gen(device, w.seed, b, h, p) for p in range(4))
    shape = (w.T, w.Hs, w.Ws, w.d)
    F = torch.randn(shape, generator=gF, device=device)
    for ax in range(3):
        F = _smooth(F, ax, w.sigma)
    F = _unit(F)
    q = _unit(F + w.qk_noise * torch.randn(shape, generator=gq, device=device))
    k = _unit(F + w.qk_noise * torch.randn(shape, generator=gk, device=device))
    v = torch.randn(shape, generator=gv, device=device)
    return q, k, v


def _video_head(w: Workload, device, b: int, h: int):
    gE, gv, gq, gk = (_gen(device, w.seed, b, h, p) for p in range(4))
    P = w.P
    nbh, nbw = w.Hs // P, w.Ws // P
    F = torch.empty((w.T, w.Hs, w.Ws, w.d), device=device)
    c = math.sqrt(1.0 - w.rho * w.rho)
    prev = None
    for t in range(w.T):
        E = torch.randn((w.Hs, w.Ws, w.d), generator=gE, device=device)
        E = _unit(_smooth(_smooth(E, 0, w.sigma), 1, w.sigma))
        prev = E if prev is None else w.rho * prev + c * E
        F[t] = prev
    # Long-range repeats: overwrite a few P x P patches with a patch from a distant frame.
    if w.copy_frac > 0:
        nb = w.T * nbh * nbw
        n_copy = int(round(w.copy_frac * nb))
        D = max(2, w.T // 4)
        src_field = F.clone()
        # Which blocks are copied is drawn on the host, so it is the same on every device.
        dst = torch.randperm(nb, generator=_gen("cpu", w.seed, b, h, 7))[:n_copy].tolist()
        gsel = _gen("cpu", w.seed, b, h, 8)
        t_of = torch.arange(nb) // (nbh * nbw)
        for j in dst:
            tj = int(t_of[j])
            cand = torch.nonzero((t_of - tj).abs() >= D).flatten()
            if cand.numel() == 0:
                continue
            s = int(cand[torch.randint(cand.numel(), (1,), generator=gsel)])
            ts, rs = divmod(s, nbh * nbw)
            hs_, ws_ = divmod(rs, nbw)
            hd_, wd_ = divmod(j % (nbh * nbw), nbw)
            F[tj, hd_ * P:(hd_ + 1) * P, wd_ * P:(wd_ + 1) * P] = \
                src_field[ts, hs_ * P:(hs_ + 1) * P, ws_ * P:(ws_ + 1) * P]
    F = _unit(F)
    if w.qk_noise > 0:
        q = _unit(F + w.qk_noise * torch.randn(F.shape, generator=gq, device=device))
        k = _unit(F + w.qk_noise * torch.randn(F.shape, generator=gk, device=device))
    else:
        q = F
        k = F
    v = torch.randn(F.shape, generator=gv, device=device)
    return q, k, v


def make_qkv(w: Workload, device: str = "cpu", heads: Optional[list] = None):
    """Q, K, V of shape [B, H, N, d] in the workload's dtype (bf16 by round-to-nearest-even).

    `heads` restricts generation to a subset of heads (the result then has
    len(heads) heads); each head's values do not depend on which others are made.
    """
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    hs = list(range(w.H)) if heads is None else list(heads)
    out = [torch.empty((w.B, len(hs), w.N, w.d), dtype=dt, device=device) for _ in range(3)]
    head_fn = _tiny_head if w.recipe == "tiny" else _video_head
    with torch.no_grad():
        for b in range(w.B):
            for hi, h in enumerate(hs):
                q, k, v = head_fn(w, device, b, h)
                for o, x in zip(out, (q, k, v)):
                    o[b, hi] = x.reshape(w.N, w.d).to(dt)
    return tuple(out)


def make_random_qkv(B, H, T, Hs, Ws, d, dtype="bf16", seed=0, device="cpu", scale=1.0):
    """Plain i.i.d. normal Q/K/V for edge-case geometries (no spatial structure)."""
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    g = torch.Generator(device=device)
    g.manual_seed(_seed_for(seed, 99, 99, 99))
    N = T * Hs * Ws
    return tuple((scale * torch.randn((B, H, N, d), generator=g, device=device)).to(dt) for _ in range(3))


def make_dout(B, H, N, d, seed=0, device="cpu"):
    """Incoming gradient dO for the backward: i.i.d. standard normal [B, H, N, d], bf16."""
    g = torch.Generator(device=device)
    g.manual_seed(_seed_for(seed, 77, 77, 77))
    return torch.randn((B, H, N, d), generator=g, device=device).to(torch.bfloat16)
