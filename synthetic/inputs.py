"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

This module draws random numbers and rounds them to the storage type; it holds
none of the method's arithmetic.  Every tensor is drawn from its own generator,
keyed by (seed, tensor name), so a tensor's values do not depend on which other
tensors were drawn before it.

Distributions (the pages ship no weights, so random-init weights of the Wan
shapes stand in): weights and biases N(0, 0.02); latents and conditioning
tokens N(0, 1).  For bf16 workloads every weight, bias and context value is
rounded to bf16 (round to nearest, ties to even) and handed to both sides as
those rounded values, so that parity measures compute error and not weight
quantisation.  Latents stay fp32 (the residual stream is fp32).

Layouts: linear weights are [in, out] (y = x @ W + b); the fused QKV weight is
[D, 3D] with column blocks (q | k | v); the cross K/V weight is [D, 2D] with
blocks (k | v); the per-block modulation table is [6, D]; the patch embedding
is [P, D] and the output head [D, P] with a [2, D] modulation table.
"""
from __future__ import annotations

import zlib
from typing import Dict

import numpy as np

from .configs import StageConfig

WEIGHT_STD = 0.02
FREQ_DIM = 256  # width of the sinusoidal timestep features


def rng_for(seed: int, tag: str) -> np.random.Generator:
    return np.random.default_rng([int(seed), zlib.crc32(tag.encode())])


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 value (ties to even), returned as fp32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32)


def _draw(cfg: StageConfig, seed: int, tag: str, shape, std: float, rounded: bool = True):
    a = rng_for(seed, tag).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if rounded and cfg.dtype == "bf16":
        a = round_bf16(a)
    return a


def block_weights(cfg: StageConfig, block: int, seed: int = 0) -> Dict[str, np.ndarray]:
    D, F = cfg.hidden, cfg.ffn
    p = f"block{block}."
    shapes = {
        "wqkv": (D, 3 * D), "bqkv": (3 * D,),
        "wo": (D, D), "bo": (D,),
        "wq2": (D, D), "bq2": (D,),
        "wkv2": (D, 2 * D), "bkv2": (2 * D,),
        "wo2": (D, D), "bo2": (D,),
        "w1": (D, F), "b1": (F,),
        "w2": (F, D), "b2": (D,),
        "tmod": (6, D),
    }
    return {k: _draw(cfg, seed, p + k, s, WEIGHT_STD) for k, s in shapes.items()}


def time_weights(cfg: StageConfig, seed: int = 0) -> Dict[str, np.ndarray]:
    """Shared timestep MLP (256 -> D -> D) and the D -> 6D modulation projection."""
    D = cfg.hidden
    shapes = {
        "wt1": (FREQ_DIM, D), "bt1": (D,),
        "wt2": (D, D), "bt2": (D,),
        "wp": (D, 6 * D), "bp": (6 * D,),
    }
    return {k: _draw(cfg, seed, "time." + k, s, WEIGHT_STD) for k, s in shapes.items()}


def head_weights(cfg: StageConfig, seed: int = 0) -> Dict[str, np.ndarray]:
    """Patch embedding (P -> D) and output head (D -> P, modulation table [2, D])."""
    D, P = cfg.hidden, cfg.latent_dim
    shapes = {"w_embed": (P, D), "b_embed": (D,), "w_head": (D, P), "b_head": (P,), "t_head": (2, D)}
    return {k: _draw(cfg, seed, "head." + k, s, WEIGHT_STD) for k, s in shapes.items()}


def latent_patches(cfg: StageConfig, stream: int, chunk: int, seed: int = 0) -> np.ndarray:
    """x^0 of one chunk as latent patches: [L, P] fp32 noise.  Stream sigma uses seed + sigma."""
    return _draw(cfg, seed + stream, f"latent_patches.c{chunk}", (cfg.tokens, cfg.latent_dim), 1.0,
                 rounded=False)


def latent(cfg: StageConfig, stream: int, chunk: int, seed: int = 0) -> np.ndarray:
    """x^0 of one chunk: [L, D] fp32 noise.  Stream sigma uses seed + sigma."""
    return _draw(cfg, seed + stream, f"latent.c{chunk}", (cfg.tokens, cfg.hidden), 1.0,
                 rounded=False)


def context(cfg: StageConfig, stream: int, seed: int = 0) -> np.ndarray:
    """Conditioning tokens of one stream: [Lc, D]."""
    return _draw(cfg, seed + stream, "context", (cfg.n_ctx, cfg.hidden), 1.0)


def hidden_rows(cfg: StageConfig, n_tasks: int, seed: int = 0, tag: str = "h_in") -> np.ndarray:
    """Stage input rows for single-stage runs: [n_tasks * L, D] fp32."""
    return _draw(cfg, seed, tag, (n_tasks * cfg.tokens, cfg.hidden), 1.0, rounded=False)


def cache_entry(cfg: StageConfig, stream: int, block: int, step: int, chunk: int,
                seed: int = 0):
    """Pre-filled noisy-KV entry (K, V), each [L, H, d], for single-stage runs."""
    shp = (cfg.tokens, cfg.heads, cfg.head_dim)
    tag = f"kv.s{stream}.b{block}.t{step}.c{chunk}"
    k = _draw(cfg, seed, tag + ".k", shp, 1.0)
    v = _draw(cfg, seed, tag + ".v", shp, 1.0)
    return k, v
