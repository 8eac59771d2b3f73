"""Seeded synthetic Q/K/V for the sampled block-sparse attention workloads.

This module only draws inputs. It holds none of the method's arithmetic and is
shared by the tests, the bench and the smoke check; the oracle never imports
it (the oracle takes arrays).

Workloads (tokens are flattened frame-major, n = (t*Y + y)*X + x):

  tiny     B=1 H=2  N=1024   grid 4x16x16  d=64  fp32, iid N(0,1), budget 25% (and 100%)
  small    B=1 H=8  N=8192   grid 8x32x32  d=128 bf16, video-shaped, budget 10%
  wan      B=1 H=40 N=75600  grid 21x45x80 d=128 bf16, video-shaped, budget 10%
  hunyuan  B=1 H=24 N=118800 grid 33x45x80 d=128 bf16, video-shaped, budget 8%
  reuse    the wan (or small) shape, four denoising steps with drifting Q/K/V,
           budgets 5/10/20%

The video-shaped generator stands in for the activations of a 720p video
diffusion transformer layer (Wan2.1: 21x45x80 latent grid, HunyuanVideo:
33x45x80), which are not available here. Per head h and channel i it draws
integer frequencies (a, b, c) in {0,1,2}^3 minus the zero vector and a phase
phi ~ U[0, 2*pi), forms f(t,y,x) = sin(2*pi*(a*t/T + b*y/Y + c*x/X) + phi), and
sets Q = 0.5*z_Q + 2*f, K = 0.5*z_K + 2*f (the same f), V = z_V with z iid
N(0,1). Values are formed in fp32 and rounded to bf16 (round to nearest even).
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

__all__ = [
    "CONFIGS", "budget_blocks", "iid_qkv", "video_qkv", "drift", "drift_device", "make_inputs",
    "sip_seed", "shape_of",
]

CONFIGS = {
    "tiny": dict(index=0, B=1, H=2, N=1024, grid=(4, 16, 16), d=64, dtype="f32",
                 budget_pct=25, kind="iid"),
    "small": dict(index=1, B=1, H=8, N=8192, grid=(8, 32, 32), d=128, dtype="bf16",
                  budget_pct=10, kind="video"),
    "wan": dict(index=2, B=1, H=40, N=75600, grid=(21, 45, 80), d=128, dtype="bf16",
                budget_pct=10, kind="video"),
    "hunyuan": dict(index=3, B=1, H=24, N=118800, grid=(33, 45, 80), d=128, dtype="bf16",
                    budget_pct=8, kind="video"),
}

REUSE_BUDGETS_PCT = (5, 10, 20)
REUSE_STEPS = 4
REUSE_SIGMA = 0.05


def budget_blocks(pct: int, M: int) -> int:
    """KV-block budget per query block: ceil(pct * M / 100) in integer arithmetic, >= 1."""
    return max(1, min(M, (pct * M + 99) // 100))


def sip_seed(step: int = 0) -> int:
    """Sampler seed used for the plan built at a given denoising step."""
    return 0x5EED0000 + step


def shape_of(name: str):
    c = CONFIGS[name]
    return c["B"], c["H"], c["N"], c["d"]


def iid_qkv(B: int, H: int, N: int, d: int, seed: int):
    """Q, K, V ~ iid N(0,1) as float32 numpy arrays of shape [B, H, N, d]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((B, H, N, d), dtype=np.float32)
    k = rng.standard_normal((B, H, N, d), dtype=np.float32)
    v = rng.standard_normal((B, H, N, d), dtype=np.float32)
    return q, k, v


def _features(grid, d, frng):
    """Low-frequency sinusoidal features [N, d] (float32) for one head."""
    T, Y, X = grid
    choices = np.array([(a, b, c) for a in range(3) for b in range(3) for c in range(3)
                        if (a, b, c) != (0, 0, 0)], dtype=np.float64)
    sel = frng.integers(0, len(choices), size=d)
    freq = choices[sel]                                   # [d, 3]
    phase = frng.uniform(0.0, 2.0 * math.pi, size=d)      # [d]
    t = np.arange(T, dtype=np.float64)[:, None, None] / T
    y = np.arange(Y, dtype=np.float64)[None, :, None] / Y
    x = np.arange(X, dtype=np.float64)[None, None, :] / X
    out = np.empty((T * Y * X, d), dtype=np.float32)
    for i in range(d):
        a, b, c = freq[i]
        ang = 2.0 * math.pi * (a * t + b * y + c * x) + phase[i]
        out[:, i] = np.sin(ang).reshape(-1)
    return out


def video_qkv(B: int, H: int, grid, d: int, seed: int, feat_seed: int,
              alpha: float = 2.0, noise: float = 0.5, threads: int = 8):
    """Video-shaped Q, K, V as bf16 CPU torch tensors of shape [B, H, N, d].

    Each (b, h) slice has its own child seed, so the result does not depend on
    the thread count.
    """
    T, Y, X = grid
    N = T * Y * X
    q = torch.empty((B, H, N, d), dtype=torch.bfloat16)
    k = torch.empty_like(q)
    v = torch.empty_like(q)
    data_children = np.random.SeedSequence(seed).spawn(B * H)
    feat_children = np.random.SeedSequence(feat_seed).spawn(H)

    def one(bh):
        b, h = divmod(bh, H)
        rng = np.random.Generator(np.random.PCG64(data_children[bh]))
        f = _features(grid, d, np.random.Generator(np.random.PCG64(feat_children[h])))
        zq = rng.standard_normal((N, d), dtype=np.float32)
        zk = rng.standard_normal((N, d), dtype=np.float32)
        zv = rng.standard_normal((N, d), dtype=np.float32)
        f *= np.float32(alpha)
        q[b, h] = torch.from_numpy(np.float32(noise) * zq + f).to(torch.bfloat16)
        k[b, h] = torch.from_numpy(np.float32(noise) * zk + f).to(torch.bfloat16)
        v[b, h] = torch.from_numpy(zv).to(torch.bfloat16)

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(one, range(B * H)))
    return q, k, v


def drift(x: torch.Tensor, seed: int, sigma: float = REUSE_SIGMA) -> torch.Tensor:
    """One denoising-step drift: x + sigma * N(0,1), rounded back to x's dtype."""
    rng = np.random.Generator(np.random.PCG64(seed))
    z = rng.standard_normal(tuple(x.shape), dtype=np.float32)
    return (x.float() + torch.from_numpy(z) * sigma).to(x.dtype)


def drift_device(x: torch.Tensor, seed: int, sigma: float = REUSE_SIGMA) -> torch.Tensor:
    """drift() drawn on x's device with torch's generator for that device
    (seeded; a different stream of numbers than drift(), for the bench's
    full-size multi-step runs, where drawing on the host would dominate)."""
    g = torch.Generator(device=x.device)
    g.manual_seed(seed)
    z = torch.randn(tuple(x.shape), generator=g, device=x.device, dtype=torch.float32)
    return (x.float() + z * sigma).to(x.dtype)


def make_inputs(name: str, threads: int = 8):
    """Inputs of a named workload: (q, k, v) as CPU torch tensors in storage dtype.

    tiny -> float32; the video-shaped workloads -> bfloat16.
    """
    c = CONFIGS[name]
    if c["kind"] == "iid":
        q, k, v = iid_qkv(c["B"], c["H"], c["N"], c["d"], seed=c["index"])
        return torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)
    return video_qkv(c["B"], c["H"], c["grid"], c["d"], seed=c["index"],
                     feat_seed=1000 + c["index"], threads=threads)
