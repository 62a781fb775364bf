"""Workload shapes for the stage-task path (no arithmetic of the method here).

A *stage task* is one DiT Transformer block at one denoising step for one latent
chunk (PhysisServe tech-report summary, AREX feed article, section "三层设计",
layer 1; 163.com release, section "PhysisServe", first bullet).  The shapes below
are the Wan-family backbones the pages evaluate (AREX article, section "实测数字":
Wan2.1 1.3B, Wan2.2 TI2V 5B, Wan2.1 14B, 4 denoising steps each) plus a tiny case
that a CPU finishes in seconds.

Both the CPU oracle and the GPU path read these records; they hold sizes only.
"""
from __future__ import annotations

import dataclasses
from typing import Tuple


@dataclasses.dataclass(frozen=True)
class StageConfig:
    name: str
    hidden: int            # D
    heads: int             # H
    head_dim: int          # d = D / H
    ffn: int               # F
    grid: Tuple[int, int, int]   # tokens of one chunk as (frames F_c, rows H_g, cols W_g)
    window: int            # W: prior chunks whose noisy KV a chunk attends to
    n_ctx: int             # Lc: conditioning tokens for cross-attention
    n_blocks: int          # B
    timesteps: Tuple[float, ...]  # t_0 > t_1 > ... > t_{S-1}; t_S = 0
    dtype: str             # "fp32" or "bf16": GEMM/attention operand type
    n_streams: int = 1
    k: int = 1             # chunks of one stream entering a step per tick
    batch: int = 1         # tasks per ps_stage_batch call in the measured run
    latent_channels: int = 16            # C of the latent video (patch embedding / output head)
    patch: Tuple[int, int, int] = (1, 2, 2)   # latent frames x rows x cols per token

    @property
    def tokens(self) -> int:
        f, h, w = self.grid
        return f * h * w

    @property
    def latent_dim(self) -> int:
        """P: latent values per token (channels x patch volume)."""
        pf, ph, pw = self.patch
        return self.latent_channels * pf * ph * pw

    @property
    def latent_shape(self) -> Tuple[int, int, int, int]:
        """(C, frames, rows, cols) of one chunk's latent."""
        (f, h, w), (pf, ph, pw) = self.grid, self.patch
        return (self.latent_channels, f * pf, h * ph, w * pw)

    @property
    def n_steps(self) -> int:
        return len(self.timesteps)

    @property
    def ring(self) -> int:
        """Ring slots per (stream, block, step): the window plus the chunks of one tick."""
        return self.window + self.k


C1 = StageConfig(
    name="c1_tiny", hidden=128, heads=2, head_dim=64, ffn=512, grid=(1, 8, 8),
    window=2, n_ctx=16, n_blocks=2, timesteps=(1.0, 0.5), dtype="fp32",
    n_streams=1, k=1, batch=2, latent_channels=8)

C2 = StageConfig(
    name="c2_wan13b_stage", hidden=1536, heads=12, head_dim=128, ffn=8960,
    grid=(1, 30, 52), window=3, n_ctx=512, n_blocks=1,
    timesteps=(1.0, 0.75, 0.5, 0.25), dtype="bf16", n_streams=1, k=1, batch=1)

C3 = StageConfig(
    name="c3_wan13b_timeshared", hidden=1536, heads=12, head_dim=128, ffn=8960,
    grid=(1, 30, 52), window=3, n_ctx=512, n_blocks=30,
    timesteps=(1.0, 0.75, 0.5, 0.25), dtype="bf16", n_streams=1, k=2, batch=8)

C4 = StageConfig(
    name="c4_wan22_5b_timeshared", hidden=3072, heads=24, head_dim=128, ffn=14336,
    grid=(1, 40, 44), window=3, n_ctx=512, n_blocks=30,
    timesteps=(1.0, 0.75, 0.5, 0.25), dtype="bf16", n_streams=1, k=2, batch=8, latent_channels=48)

C5 = StageConfig(
    name="c5_wan14b_stage16", hidden=5120, heads=40, head_dim=128, ffn=13824,
    grid=(1, 30, 52), window=3, n_ctx=512, n_blocks=1,
    timesteps=(1.0, 0.75, 0.5, 0.25), dtype="bf16", n_streams=16, k=1, batch=16)

CONFIGS = {c.name: c for c in (C1, C2, C3, C4, C5)}
SHORT = {"c1": C1, "c2": C2, "c3": C3, "c4": C4, "c5": C5}


def get(name: str) -> StageConfig:
    if name in SHORT:
        return SHORT[name]
    return CONFIGS[name]


def with_(cfg: StageConfig, **kw) -> StageConfig:
    """A copy with some fields replaced (reduced depth, fewer streams, ...)."""
    return dataclasses.replace(cfg, **kw)


def stage_flops(cfg: StageConfig, n_read: int | None = None) -> float:
    """Algorithmic FLOPs of one stage task with a full window.

    Counts QKV, self-attention over (n_read + 1) chunks, O, cross-Q,
    cross-attention, cross-O and the FFN.  The cross K/V projection is cached
    per (stream, block) and not counted; softmax and elementwise work are not
    counted.
    """
    L, D, F, Lc = cfg.tokens, cfg.hidden, cfg.ffn, cfg.n_ctx
    nr = cfg.window if n_read is None else n_read
    return (2 * L * D * 3 * D + 4 * L * (nr + 1) * L * D + 2 * L * D * D
            + 2 * L * D * D + 4 * L * Lc * D + 2 * L * D * D + 4 * L * D * F)
