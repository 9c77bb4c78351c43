"""The five synthetic workloads the path is checked and measured on.

Shapes follow the pages' workloads: FLUX.1-dev latents at 1024^2, 2048^2 and 4096^2
(16x16 latent patches -> 64x64, 128x128, 256x256 token grids, 24 heads of 128), a
Wan2.1-shaped video latent (21 frames of 30x52 tokens, 12 heads of 128), the pages' own
Wan measurement grid (21 frames of 60x104 tokens), plus a tiny fp32 2-D case small
enough for exhaustive checks. Each workload lists the shifts of
its block cycle: the path is called once per shift on the same q, k, v.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" or "bf16"
    batch: int
    heads: int
    head_dim: int
    grid: Tuple[int, int, int]     # (T, H, W) token grid
    window: Tuple[int, int, int]   # (wt, wh, ww)
    shifts: Tuple[Tuple[int, int, int], ...]
    seed: int

    @property
    def tokens(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def window_tokens(self) -> int:
        a, b, c = self.window
        return a * b * c

    @property
    def num_windows(self) -> int:
        return self.tokens // self.window_tokens

    @property
    def shape(self):
        return (self.batch, self.heads, self.tokens, self.head_dim)

    def window_flops(self) -> int:
        """4*B*heads*N*W*d: QK^T and PV, two flops per multiply-add."""
        return 4 * self.batch * self.heads * self.tokens * self.window_tokens * self.head_dim

    def full_flops(self) -> int:
        return 4 * self.batch * self.heads * self.tokens * self.tokens * self.head_dim

    def io_bytes(self) -> int:
        """q, k, v read once and out written once."""
        elem = 2 if self.dtype == "bf16" else 4
        return 4 * self.batch * self.heads * self.tokens * self.head_dim * elem


WORKLOADS = (
    Workload("tiny-2d-16x16-w8", "f32", 1, 2, 64, (1, 16, 16), (1, 8, 8),
             ((0, 0, 0), (0, 4, 4)), 1),
    Workload("flux-1024-64x64-w16", "bf16", 1, 24, 128, (1, 64, 64), (1, 16, 16),
             ((0, 0, 0), (0, 8, 8)), 2),
    Workload("flux-2048-128x128-w32", "bf16", 1, 24, 128, (1, 128, 128), (1, 32, 32),
             ((0, 0, 0), (0, 16, 16)), 3),
    Workload("flux-4096-256x256-w32", "bf16", 1, 24, 128, (1, 256, 256), (1, 32, 32),
             ((0, 0, 0), (0, 16, 0), (0, 0, 16), (0, 16, 16)), 4),
    Workload("wan-21x30x52-w7x15x26", "bf16", 1, 12, 128, (21, 30, 52), (7, 15, 26),
             ((0, 0, 0), (3, 7, 13)), 5),
    # The pages' own Wan measurement shape (Table 3): 1664x960 output, 81 frames -> a
    # 21x60x104 latent grid; windows keep the whole temporal axis (21) with 15x26 spatial
    # extent, i.e. 16 windows of 8190 tokens.
    Workload("wan-21x60x104-w21x15x26", "bf16", 1, 12, 128, (21, 60, 104), (21, 15, 26),
             ((0, 0, 0), (0, 7, 13)), 6),
)

BY_NAME = {w.name: w for w in WORKLOADS}
