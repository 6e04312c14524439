"""Workload shapes and seeded synthetic inputs.

This module holds only shapes and random draws: none of the attention
arithmetic.  Both the GPU path's tests/bench and the CPU oracle's tests take
their inputs from here.

Shapes follow the video latents the pages work at: a 720P clip for sliding
tile attention (Sliding Tile Attention, abstract: a 5-second 720P video), and
1080P / 2K / 4K latents for the global-local decomposition (UltraGen summary,
§5.2 and App. C).  Every tensor is logically [B, heads, N, D] with the token
axis in raster order n = (t*H + h)*W + w.

Recipe (fixed, so any run regenerates identical inputs):
  * a ``torch.Generator`` on the target device, seeded with
    ``seed_for(workload, tensor_id)``; tensor ids 0=Q, 1=K, 2=V, 3=gate,
    4=outlier rows;
  * Q, K, V: fp32 standard normal of shape [B, heads, N, D], then rounded to
    the workload dtype (bf16 by round-to-nearest-even);
  * outlier rows (2K workload): per (b, h), floor(frac * N) distinct token
    rows chosen by ``randperm`` are multiplied by ``outlier_scale`` before the
    bf16 rounding (x8 is exact in bf16);
  * gate: one U(0, 1) value per head, fp32.
"""
from __future__ import annotations

import dataclasses
import zlib
from typing import Optional, Tuple

import torch

Triple = Tuple[int, int, int]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    grid: Triple                     # (T, H, W) latent tokens
    heads: int
    head_dim: int
    dtype: str                       # "f32" | "bf16"
    tile: Triple                     # tile extent in tokens per dim
    window: Triple                   # window extent in tiles per dim (odd)
    shifts: Tuple[Triple, ...] = ((0, 0, 0),)   # one local call per shift
    pool_hw: Optional[Tuple[int, int]] = None   # global branch pooling
    batch: int = 1
    scale: Optional[float] = None    # None -> 1/sqrt(head_dim)
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    description: str = ""

    @property
    def n_tokens(self) -> int:
        T, H, W = self.grid
        return T * H * W

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else self.head_dim ** -0.5

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


# The five workloads: tiny fp32, 720P STA, 1080P dual-branch, 4K local+global,
# 2K cross-window pair.
WORKLOADS = {
    "tiny_f32": Workload(
        "tiny_f32", (4, 8, 8), heads=2, head_dim=64, dtype="f32",
        tile=(2, 4, 4), window=(3, 3, 3), scale=1.0 / 8.0,
        description="T=4,H=8,W=8, tile 2x4x4, window 3x3x3 tiles, 2 heads, d=64, fp32"),
    "sta_720p": Workload(
        "sta_720p", (30, 48, 80), heads=24, head_dim=128, dtype="bf16",
        tile=(6, 8, 8), window=(3, 3, 5),
        description="720P latent T=30,H=48,W=80, tile 6x8x8, window 3x3x5 tiles, 24 heads, d=128, bf16"),
    "dual_1080p": Workload(
        "dual_1080p", (21, 68, 120), heads=24, head_dim=128, dtype="bf16",
        tile=(21, 17, 30), window=(1, 1, 1), pool_hw=(4, 4),
        description="1080P latent T=21,H=68,W=120; local 17x30 spatial windows over all frames; "
                    "global over 4x4-pooled K/V; gated sum"),
    "local_global_4k": Workload(
        "local_global_4k", (21, 136, 240), heads=24, head_dim=128, dtype="bf16",
        tile=(3, 8, 8), window=(3, 5, 5), pool_hw=(8, 8),
        description="4K latent T=21,H=136,W=240, tile 3x8x8, window 3x5x5 tiles; "
                    "global over 8x8-pooled K/V; gated sum"),
    "cross_window_2k": Workload(
        "cross_window_2k", (21, 90, 160), heads=16, head_dim=128, dtype="bf16",
        tile=(4, 8, 8), window=(1, 1, 1), shifts=((0, 0, 0), (2, 4, 4)),
        outlier_frac=0.05, outlier_scale=8.0,
        description="2K latent T=21,H=90,W=160, tile 4x8x8 (partial edge tiles), window 1 tile, "
                    "unshifted then half-tile-shifted call pair, 16 heads, 5% of K rows x8"),
}


def seed_for(workload_name: str, tensor_id: int, base_seed: int = 0) -> int:
    """Deterministic 63-bit seed per (workload, tensor, base seed)."""
    h = zlib.crc32(f"{workload_name}/{tensor_id}/{base_seed}".encode())
    return (h << 16) ^ (tensor_id * 0x9E3779B1) ^ base_seed


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def make_qkv(w: Workload, device="cpu", base_seed: int = 0, layout: str = "bhnd"):
    """Seeded Q, K, V for workload ``w`` (see module docstring for the recipe).

    ``layout`` "bhnd" gives contiguous [B, heads, N, D]; "bnhd" gives a
    [B, heads, N, D] view of contiguous [B, N, heads, D] storage.
    """
    shape = (w.batch, w.heads, w.n_tokens, w.head_dim)
    out = []
    for tid in range(3):
        g = _gen(device, seed_for(w.name, tid, base_seed))
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if tid == 1 and w.outlier_frac > 0:
            go = _gen(device, seed_for(w.name, 4, base_seed))
            count = int(w.outlier_frac * w.n_tokens)
            for b in range(w.batch):
                for h in range(w.heads):
                    rows = torch.randperm(w.n_tokens, generator=go, device=device)[:count]
                    x[b, h, rows] *= w.outlier_scale
        x = x.to(w.torch_dtype)
        if layout == "bnhd":
            x = x.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        out.append(x)
    return tuple(out)


def make_gate(w: Workload, device="cpu", base_seed: int = 0) -> torch.Tensor:
    """Per-head U(0, 1) gate, fp32 [heads]."""
    g = _gen(device, seed_for(w.name, 3, base_seed))
    return torch.rand((w.heads,), generator=g, device=device, dtype=torch.float32)


def make_tensor(shape, dtype, device="cpu", seed: int = 0, scale: float = 1.0):
    """Generic seeded N(0, scale^2) tensor for small ad-hoc test shapes."""
    g = _gen(device, seed)
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32) * scale
    return x.to(dtype)
