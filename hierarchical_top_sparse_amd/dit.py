"""A synthetic Pixel-DiT-S training step with LLSA as its attention.

The pages train "Pixel DiT-S" on FFHQ with patch size 1x1 (every pixel is a token; summary
sec. 5.1-5.2, Table 2) and report its training throughput with LLSA against full attention.
This module builds that architecture with random weights and synthetic data, so that the op
can be timed inside the network it was made for: no dataset and no trained weights.

Architecture (DiT-S: hidden 384, 6 heads of 64, MLP ratio 4, adaptive layer norm):
  * pixels [b, 3, H, W] -> tokens by a per-pixel linear map (a 1x1 patch embedding), plus a
    fixed 2D sine-cosine position embedding;
  * conditioning c = timestep embedding (sinusoidal features -> MLP) + class embedding;
  * each block: x += g1 * attn(mod(LN(x), s1, t1)); x += g2 * mlp(mod(LN(x), s2, t2)), with the
    six modulation vectors produced from c by SiLU + linear (adaLN);
  * attention: QKV projection, then LLSA (or the library's dense attention for the
    full-attention baseline), then the output projection;
  * final layer: adaLN-modulated LN and a linear map back to 3 channels per pixel.
The token order is hoisted to the network's entry: the tokens are permuted once into Morton
order after the embedding, every block runs LLSA with layout LLSA_LAYOUT_MORTON (no
reorder inside the op), and the output is permuted back once at the end.  Everything but the
attention is per token, so the network's result does not depend on this order.
"""
from __future__ import annotations

import math

import torch
import torch.nn as nn
import torch.nn.functional as F

from . import ops


def morton_permutation(height: int, width: int) -> torch.Tensor:
    """perm[m] = raster index of the m-th token along the Z-order curve (x bits in the even
    positions of m, y bits in the odd ones, the longer side's extra bits on top)."""
    hb, wb = height.bit_length() - 1, width.bit_length() - 1
    m = torch.arange(height * width, dtype=torch.int64)
    x = torch.zeros_like(m)
    y = torch.zeros_like(m)
    pos = 0
    for i in range(max(hb, wb)):
        if i < wb:
            x |= ((m >> pos) & 1) << i
            pos += 1
        if i < hb:
            y |= ((m >> pos) & 1) << i
            pos += 1
    return y * width + x


def sincos_2d(height: int, width: int, dim: int) -> torch.Tensor:
    """Fixed 2D sine-cosine position embedding [height*width, dim] in raster order."""
    def one(pos, d):
        omega = 1.0 / 10000 ** (torch.arange(d // 2, dtype=torch.float64) / (d / 2))
        out = pos[:, None].double() * omega[None]
        return torch.cat([out.sin(), out.cos()], dim=1)
    yy, xx = torch.meshgrid(torch.arange(height), torch.arange(width), indexing="ij")
    return torch.cat([one(yy.reshape(-1), dim // 2), one(xx.reshape(-1), dim // 2)],
                     dim=1).float()


def timestep_features(t: torch.Tensor, dim: int = 256) -> torch.Tensor:
    half = dim // 2
    freqs = torch.exp(-math.log(10000) * torch.arange(half, device=t.device) / half)
    args = t.float()[:, None] * freqs[None]
    return torch.cat([torch.cos(args), torch.sin(args)], dim=1)


def modulate(x, shift, scale):
    return x * (1 + scale[:, None]) + shift[:, None]


class Attention(nn.Module):
    """QKV projection -> LLSA (or dense attention) -> output projection, on [b, N, C]."""

    def __init__(self, dim, heads, height, width, mode="llsa", levels=3, topk=8, block=16,
                 layout=ops.LLSA_LAYOUT_MORTON):
        super().__init__()
        self.heads, self.hw, self.mode = heads, (height, width), mode
        self.levels, self.topk, self.block, self.layout = levels, topk, block, layout
        self.qkv = nn.Linear(dim, 3 * dim)
        self.proj = nn.Linear(dim, dim)

    def forward(self, x):
        b, n, c = x.shape
        qkv = self.qkv(x).view(b, n, 3, self.heads, c // self.heads).permute(2, 0, 3, 1, 4)
        q, k, v = (t.contiguous() for t in qkv)   # [b, H, N, 64] each
        if self.mode == "llsa":
            o = ops.llsa_attention(q, k, v, *self.hw, self.levels, self.topk,
                                   layout=self.layout, block=self.block)
        else:
            o = ops.dense_attention(q, k, v)
        return self.proj(o.transpose(1, 2).reshape(b, n, c))


class Block(nn.Module):
    def __init__(self, dim, heads, height, width, **attn):
        super().__init__()
        self.norm1 = nn.LayerNorm(dim, elementwise_affine=False, eps=1e-6)
        self.attn = Attention(dim, heads, height, width, **attn)
        self.norm2 = nn.LayerNorm(dim, elementwise_affine=False, eps=1e-6)
        self.mlp = nn.Sequential(nn.Linear(dim, 4 * dim), nn.GELU(approximate="tanh"),
                                 nn.Linear(4 * dim, dim))
        self.ada = nn.Sequential(nn.SiLU(), nn.Linear(dim, 6 * dim))

    def forward(self, x, c):
        s1, t1, g1, s2, t2, g2 = self.ada(c).chunk(6, dim=1)
        x = x + g1[:, None] * self.attn(modulate(self.norm1(x), s1, t1))
        return x + g2[:, None] * self.mlp(modulate(self.norm2(x), s2, t2))


class PixelDiT(nn.Module):
    """Pixel DiT with 1x1 patches: depth 12, hidden 384, 6 heads is DiT-S."""

    def __init__(self, height, width, depth=12, dim=384, heads=6, classes=1, mode="llsa",
                 levels=3, topk=8, block=16, hoist_reorder=True):
        super().__init__()
        layout = ops.LLSA_LAYOUT_MORTON if hoist_reorder else ops.LLSA_LAYOUT_RASTER
        self.hoist = hoist_reorder
        self.hw = (height, width)
        self.embed = nn.Linear(3, dim)
        self.t_mlp = nn.Sequential(nn.Linear(256, dim), nn.SiLU(), nn.Linear(dim, dim))
        self.y_embed = nn.Embedding(classes, dim)
        perm = morton_permutation(height, width)
        pos = sincos_2d(height, width, dim)
        self.register_buffer("perm", perm, persistent=False)
        self.register_buffer("inv_perm", torch.argsort(perm), persistent=False)
        self.register_buffer("pos", pos[perm] if hoist_reorder else pos, persistent=False)
        self.blocks = nn.ModuleList(
            Block(dim, heads, height, width, mode=mode, levels=levels, topk=topk, block=block,
                  layout=layout) for _ in range(depth))
        self.norm = nn.LayerNorm(dim, elementwise_affine=False, eps=1e-6)
        self.ada = nn.Sequential(nn.SiLU(), nn.Linear(dim, 2 * dim))
        self.out = nn.Linear(dim, 3)

    def forward(self, img, t, y):
        b = img.shape[0]
        tok = img.flatten(2).transpose(1, 2)                  # [b, N, 3], raster order
        if self.hoist:
            tok = tok[:, self.perm]                            # Morton order, once
        x = self.embed(tok) + self.pos
        c = self.t_mlp(timestep_features(t)) + self.y_embed(y)
        for blk in self.blocks:
            x = blk(x, c)
        shift, scale = self.ada(c).chunk(2, dim=1)
        x = self.out(modulate(self.norm(x), shift, scale))     # [b, N, 3]
        if self.hoist:
            x = x[:, self.inv_perm]
        return x.transpose(1, 2).reshape(b, 3, *self.hw)


def synthetic_batch(batch, height, width, device, seed=0):
    """Noisy images, noise targets, timesteps and class labels, seeded (no dataset)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    x0 = torch.rand(batch, 3, height, width, generator=g) * 2 - 1
    noise = torch.randn(batch, 3, height, width, generator=g)
    t = torch.randint(0, 1000, (batch,), generator=g)
    a = torch.cos(t.float() / 1000 * math.pi / 2)[:, None, None, None]
    xt = a * x0 + (1 - a * a).sqrt() * noise
    y = torch.zeros(batch, dtype=torch.int64)
    return tuple(z.to(device) for z in (xt, noise, t, y))


def train_step(model, opt, batch):
    """One training step: forward (bf16 autocast), noise-prediction MSE, backward, AdamW."""
    xt, noise, t, y = batch
    opt.zero_grad(set_to_none=True)
    with torch.autocast(device_type="cuda", dtype=torch.bfloat16):
        pred = model(xt, t, y)
    loss = F.mse_loss(pred.float(), noise)
    loss.backward()
    opt.step()
    return loss
