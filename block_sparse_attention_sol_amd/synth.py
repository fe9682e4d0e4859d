"""Seeded synthetic video-token inputs (Q, K, V) for the Sol-Attn forward pass.

This module holds the input recipe only -- no step of the attention method.  Both the GPU path
and the CPU oracle consume what it produces; it imports neither of them (numpy and torch only).

Recipe (one attention head at a time, numpy PCG64 seeded once per workload):
  * tokens sit on a T x Hg x W latent grid, flattened row-major: n = (t*Hg + y)*W + x;
  * a smooth positional field P, shared by Q, K and V of the head, is a sum of 8 sinusoids per
    channel with random frequencies f in [0, 3) cycles per grid extent on each axis and random
    phases: P[n, c] = A * sqrt(2/8) * sum_m sin(2 pi (f0 t/T + f1 y/Hg + f2 x/W) + phase), so the
    per-channel RMS of P is about A;
  * Q, K, V = standard normal noise (float32, drawn in that order) + P;
  * everything is rounded to bf16 (round-to-nearest-even) at the end.
Draw order: (long-video workload only) the per-head amplitudes A ~ U(lo, hi) for all heads first;
then per head: f (8, d, 3), phases (8, d), noise Q, noise K, noise V.

The pages (video DiTs: Wan2.1-14B, HunyuanVideo, LTX) give no tensors; these inputs stand in for
those models' attention inputs at their latent-grid token counts.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    d: int
    grid: tuple          # (T, Hg, W)
    block: int
    amp: float = 1.0     # RMS amplitude of the positional field
    amp_range: tuple | None = None   # per-head amplitude ~ U(lo, hi) instead of amp
    betas: tuple = ()    # fixed beta values for this workload (empty: beta is tuned)
    target_density: tuple = ()       # kept-tile densities beta is tuned to

    @property
    def N(self) -> int:
        T, Hg, W = self.grid
        return T * Hg * W

    @property
    def M(self) -> int:
        return (self.N + self.block - 1) // self.block


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 64, (4, 16, 16), 64, amp=1.0, betas=(0.5,)),
    "ltx": Workload("ltx", 1, 32, 64, (8, 24, 32), 64, amp=1.5, betas=(0.0, 0.5, 1.0, 1.5)),
    "wan": Workload("wan", 1, 40, 128, (21, 45, 80), 128, amp=2.0, target_density=(0.15,)),
    "hunyuan": Workload("hunyuan", 1, 24, 128, (33, 45, 80), 128, amp=2.0,
                        target_density=(0.10, 0.15, 0.25)),
    "long": Workload("long", 1, 40, 128, (61, 45, 80), 128, amp_range=(1.0, 3.0),
                     target_density=(0.08,)),
}


def positional_field(rng: np.random.Generator, grid: tuple, d: int, amp: float) -> np.ndarray:
    """Draw f and phases from rng and return P [N, d] float64 (see module docstring).

    Evaluated separably: with a = 2 pi f0 t/T + phase and b = 2 pi (f1 y/Hg + f2 x/W),
    sin(a + b) = sin a cos b + cos a sin b, so each channel is a (T x 16) @ (16 x Hg*W) product."""
    T, Hg, W = grid
    f = rng.uniform(0.0, 3.0, (8, d, 3))
    ph = rng.uniform(0.0, 2.0 * math.pi, (8, d))
    t = np.arange(T, dtype=np.float64) / T
    y = np.arange(Hg, dtype=np.float64) / Hg
    x = np.arange(W, dtype=np.float64) / W
    # a[c, t, m], b[c, m, yx]
    a = 2.0 * math.pi * f[:, :, 0].T[:, None, :] * t[None, :, None] + ph.T[:, None, :]
    b = 2.0 * math.pi * (f[:, :, 1].T[:, :, None, None] * y[None, None, :, None]
                         + f[:, :, 2].T[:, :, None, None] * x[None, None, None, :])
    b = b.reshape(d, 8, Hg * W)
    lhs = np.concatenate([np.sin(a), np.cos(a)], axis=2)            # [d, T, 16]
    rhs = np.concatenate([np.cos(b), np.sin(b)], axis=1)            # [d, 16, HW]
    P = np.matmul(lhs, rhs)                                         # [d, T, HW]
    return (amp * math.sqrt(2.0 / 8.0)) * P.reshape(d, T * Hg * W).T


def head_arrays(rng: np.random.Generator, grid: tuple, d: int, amp: float):
    """One head: (q, k, v) float32 [N, d] before bf16 rounding."""
    T, Hg, W = grid
    N = T * Hg * W
    P = positional_field(rng, grid, d, amp).astype(np.float32)
    q = rng.standard_normal((N, d), dtype=np.float32)
    q += P
    k = rng.standard_normal((N, d), dtype=np.float32)
    k += P
    v = rng.standard_normal((N, d), dtype=np.float32)
    v += P
    return q, k, v


def amplitudes(w: Workload, rng: np.random.Generator) -> np.ndarray:
    if w.amp_range is not None:
        return rng.uniform(w.amp_range[0], w.amp_range[1], w.H)
    return np.full(w.H, w.amp)


def generate(w: Workload | str, seed: int = 0, heads: int | None = None, keep_fp32: bool = False,
             progress=None):
    """Q, K, V as bf16 torch CPU tensors [B, H, N, d] (contiguous).

    heads: generate only the first `heads` heads (the draw sequence of those heads is identical
    to a full generation).  keep_fp32: also return the fp32 arrays before rounding.
    progress: optional callable(b, h) invoked after each head is generated."""
    import torch

    if isinstance(w, str):
        w = WORKLOADS[w]
    H = w.H if heads is None else min(heads, w.H)
    rng = np.random.default_rng(seed)
    A = amplitudes(w, rng)
    N, d = w.N, w.d
    out = [torch.empty((w.B, H, N, d), dtype=torch.bfloat16) for _ in range(3)]
    masters = [np.empty((w.B, H, N, d), np.float32) for _ in range(3)] if keep_fp32 else None
    for b in range(w.B):
        for h in range(H):
            arrs = head_arrays(rng, w.grid, d, float(A[h]))
            for i, a in enumerate(arrs):
                out[i][b, h].copy_(torch.from_numpy(a).to(torch.bfloat16))
                if keep_fp32:
                    masters[i][b, h] = a
            if progress is not None:
                progress(b, h)
    if keep_fp32:
        return out[0], out[1], out[2], masters
    return out[0], out[1], out[2]


def random_qkv(B: int, H: int, N: int, d: int, seed: int = 0, scale: float = 1.0):
    """Plain N(0, scale^2) bf16 tensors [B, H, N, d] (edge-case shapes for tests)."""
    import torch

    rng = np.random.default_rng(seed)
    t = [torch.from_numpy((scale * rng.standard_normal((B, H, N, d))).astype(np.float32))
         .to(torch.bfloat16) for _ in range(3)]
    return t[0], t[1], t[2]


def anisotropic_qkv(B: int, H: int, N: int, d: int, seed: int = 0, strength: float = 24.0,
                    noise: float = 0.5, leak: float = 0.02):
    """Keys with one strong shared direction, queries nearly orthogonal to it (bf16 tensors
    [B, H, N, d]): a hard case for the proxy-row statistics.

    Per head: a random unit direction u (not aligned with any axis); K = noise * N(0, 1)
    + c_n u with c_n = strength * sin(2 pi * 3 n / N + phase), so block means of K vary strongly
    along u from block to block; Q = N(0, 1) with its component along u replaced by
    leak * N(0, 1); V = N(0, 1).  The proxy rows then have a small spread set by the noise,
    beside a pooled-key covariance whose largest eigenvalue is strength^2 / 2."""
    import torch

    rng = np.random.default_rng(seed)
    q = np.empty((B, H, N, d), np.float32)
    k = np.empty_like(q)
    v = np.empty_like(q)
    n = np.arange(N, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            u = rng.standard_normal(d)
            u /= np.linalg.norm(u)
            c = strength * np.sin(2.0 * math.pi * 3.0 * n / N + rng.uniform(0.0, 2.0 * math.pi))
            k[b, h] = noise * rng.standard_normal((N, d)) + c[:, None] * u[None, :]
            qq = rng.standard_normal((N, d))
            qq -= (qq @ u)[:, None] * u[None, :]
            qq += leak * rng.standard_normal(N)[:, None] * u[None, :]
            q[b, h] = qq
            v[b, h] = rng.standard_normal((N, d))
    return tuple(torch.from_numpy(x).to(torch.bfloat16) for x in (q, k, v))
