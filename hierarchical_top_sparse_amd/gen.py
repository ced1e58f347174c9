"""Seeded synthetic inputs for LLSA: pixel-token Q, K, V and the upstream gradient dO.

This module holds only input generation. It does none of the method's arithmetic, so both
the HIP path and the CPU oracle may consume what it produces.

Recipe (the pages train pixel-space DiTs on face and ImageNet images, which are not
available here; these fields stand in for the smooth, spatially correlated activations such
models see):

* Q and K, independently per (batch, head, channel): a smooth 2D field
  F(y, x) = sum_{m<8} sin(2*pi*(u_m*x/W + v_m*y/H) + phi_m) with integer frequencies
  (u_m, v_m) uniform in [-4, 4]^2 minus (0, 0) and phases uniform in [0, 2*pi), plus
  0.5 * N(0, 1) noise per token and channel.
* V ~ N(0, 1) and dO ~ N(0, 1).
* Generated in float32 and rounded once (round-to-nearest-even) to the requested dtype.

Tokens are in raster order: token t = y * width + x, tensors are [batch, heads, N, head_dim].
"""
from __future__ import annotations

import numpy as np
import torch

TENSOR_IDS = {"q": 1, "k": 2, "v": 3, "do": 4}
N_WAVES = 8
MAX_FREQ = 4
NOISE_STD = 0.5


def _smooth_fields(rng: np.random.Generator, n_fields: int, height: int, width: int) -> np.ndarray:
    """n_fields independent sums of N_WAVES low-frequency sinusoids, shape [n_fields, H*W]."""
    u = rng.integers(-MAX_FREQ, MAX_FREQ + 1, size=(n_fields, N_WAVES))
    v = rng.integers(-MAX_FREQ, MAX_FREQ + 1, size=(n_fields, N_WAVES))
    zero = (u == 0) & (v == 0)
    while zero.any():
        u[zero] = rng.integers(-MAX_FREQ, MAX_FREQ + 1, size=int(zero.sum()))
        v[zero] = rng.integers(-MAX_FREQ, MAX_FREQ + 1, size=int(zero.sum()))
        zero = (u == 0) & (v == 0)
    phi = rng.uniform(0.0, 2.0 * np.pi, size=(n_fields, N_WAVES))
    xs = np.arange(width, dtype=np.float64) / width
    ys = np.arange(height, dtype=np.float64) / height
    # sin(a + b) = sin(a)cos(b) + cos(a)sin(b), with a over x and b over y (incl. phase):
    ax = 2.0 * np.pi * u[:, :, None] * xs[None, None, :]                      # [F, M, W]
    by = 2.0 * np.pi * v[:, :, None] * ys[None, None, :] + phi[:, :, None]    # [F, M, H]
    left = np.concatenate([np.cos(by), np.sin(by)], axis=1).transpose(0, 2, 1)  # [F, H, 2M]
    right = np.concatenate([np.sin(ax), np.cos(ax)], axis=1)                   # [F, 2M, W]
    field = np.matmul(left, right)                                             # [F, H, W]
    return field.reshape(n_fields, height * width)


def field_plus_noise(seed: int, batch: int, heads: int, height: int, width: int,
                     head_dim: int) -> np.ndarray:
    """Smooth field + 0.5*N(0,1) noise, float32 [batch, heads, N, head_dim]."""
    rng = np.random.default_rng(seed)
    n = height * width
    out = np.empty((batch, heads, n, head_dim), dtype=np.float32)
    for b in range(batch):
        for h in range(heads):
            f = _smooth_fields(rng, head_dim, height, width)        # [d, N]
            noise = rng.standard_normal((n, head_dim), dtype=np.float32)
            out[b, h] = f.T.astype(np.float32) + np.float32(NOISE_STD) * noise
    return out


def gaussian(seed: int, batch: int, heads: int, n: int, head_dim: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.standard_normal((batch, heads, n, head_dim), dtype=np.float32)


def to_dtype(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """Round a float32 array once to `dtype` (RNE for bfloat16) as a CPU tensor."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype)


def make_inputs(batch: int, heads: int, height: int, width: int, head_dim: int = 64,
                dtype: torch.dtype = torch.bfloat16, seed_base: int = 0,
                with_grad: bool = False) -> dict:
    """Seeded raster-order inputs.

    Returns {"q","k","v"[, "do"]} as CPU tensors of `dtype`; the exact values the oracle
    must read are `t.double().numpy()` of those tensors.  Seeds are seed_base + tensor id.
    """
    n = height * width
    out = {
        "q": to_dtype(field_plus_noise(seed_base + TENSOR_IDS["q"], batch, heads, height, width,
                                       head_dim), dtype),
        "k": to_dtype(field_plus_noise(seed_base + TENSOR_IDS["k"], batch, heads, height, width,
                                       head_dim), dtype),
        "v": to_dtype(gaussian(seed_base + TENSOR_IDS["v"], batch, heads, n, head_dim), dtype),
    }
    if with_grad:
        out["do"] = to_dtype(gaussian(seed_base + TENSOR_IDS["do"], batch, heads, n, head_dim),
                             dtype)
    return out


# The five workloads the measurements are quoted on (all head_dim 64, B=16, K=8).
CONFIGS = {
    "tiny64": dict(batch=1, heads=2, height=64, width=64, levels=2, dtype=torch.float32,
                   backward=False, seed_base=0),
    "ffhq128": dict(batch=4, heads=6, height=128, width=128, levels=2, dtype=torch.bfloat16,
                    backward=False, seed_base=1000),
    "px256": dict(batch=1, heads=6, height=256, width=256, levels=3, dtype=torch.bfloat16,
                  backward=False, seed_base=2000),
    "px256_train": dict(batch=2, heads=6, height=256, width=256, levels=3,
                        dtype=torch.bfloat16, backward=True, seed_base=3000),
    "px512_train": dict(batch=1, heads=6, height=512, width=512, levels=3,
                        dtype=torch.bfloat16, backward=True, seed_base=4000),
}
