"""The Wan-shaped workloads the library is tested and measured on.

Shapes come from the model configurations on the pages ("Wan2.2 code
walkthrough": A14B dim 5120 / 40 heads, TI2V-5B dim 3072 / 24 heads;
1.3B dim 1536 / 12 heads; head size 128; 512 umT5 text tokens) and the token
grids of the clip sizes: latent (1 + (frames-1)/4) x H/8 x W/8 (x H/16 x W/16
for the TI2V VAE), then 1x2x2 patches.
"""

from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    batch: int
    grid: tuple          # (f, h, w) latent-patch grid
    heads: int
    text_len: int
    head_dim: int = 128
    eps: float = 1e-6
    rope_theta: float = 10000.0

    @property
    def tokens(self) -> int:
        f, h, w = self.grid
        return f * h * w

    @property
    def dim(self) -> int:
        return self.heads * self.head_dim

    def self_attn_flop(self) -> float:
        """4 * L^2 * d * H * B: two L x L x d products per (batch, head)."""
        return 4.0 * self.tokens ** 2 * self.head_dim * self.heads * self.batch

    def cross_attn_flop(self) -> float:
        return 4.0 * self.tokens * self.text_len * self.head_dim * self.heads * self.batch


WORKLOADS = [
    Workload(1, "tiny-5x8x8", 1, (5, 8, 8), 2, 32),
    Workload(2, "wan1.3b-480p", 1, (21, 30, 52), 12, 512),
    Workload(3, "a14b-480p", 1, (21, 30, 52), 40, 512),
    Workload(4, "ti2v5b-720p", 1, (31, 22, 40), 24, 512),
    Workload(5, "a14b-720p-cfg", 2, (21, 45, 80), 40, 512),
]

BY_NAME = {w.name: w for w in WORKLOADS}
