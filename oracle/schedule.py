"""Chunk x step schedules over the noisy-KV ring (oracle, float64).

Sources: each chunk starts from pure noise and goes through S denoising steps;
chunk c+1 need not wait for chunk c to finish all of its steps -- it reads the
noisy KV chunk c left at the same step, so adjacent chunks' denoising is offset
and overlaps (AREX feed article, section "难题"; 163.com release, section
"新一代物理 AI 的基础设施", Fig. 1 right).  Stages on one GPU batch tasks of
the same block from different chunks and steps (AREX article, section
"三层设计", layer 2; 163.com release, bullet "时分复用", Fig. 3).

Two schedules compute the same thing:
  * sequential: for stream, for chunk, for step, for block -- one task at a time;
  * staggered: tick tau holds the tasks (stream, c, s) with c = k (tau - s) + j,
    0 <= j < k; for each block every task of the tick forms one batch; inside a
    batch all KV writes come before any attention read (so chunk c + 1 can read
    what chunk c wrote in the same batch); after the last block each task of the
    tick takes its Euler step.
Because batching and staggering only reorder independent work, the two must
give bitwise identical latents and caches; the tests assert exactly that.

Euler step of flow matching: x^{s+1} = x^s - (t_s - t_{s+1}) v with
t_S = 0 and v the velocity prediction: the output of the last block, or, with
the patch embedding and output head, x holds the chunk's latent patches,
h_0 = patch_embed(x) and v = output_head(h_B, u(t_s)) (``head.py``).
"""
from __future__ import annotations

import math
from typing import Callable, Dict, List, Sequence, Tuple

import numpy as np

from .block import F64, context_kv, modulation, qkv_phase, rest_phase, time_embedding
from .head import output_head, patch_embed, time_mlp


def shifted_timesteps(n_steps: int, shift: float = 1.0) -> tuple:
    """t_0 > ... > t_{S-1} of an S-step sampler: the uniform grid u_s = 1 - s/S
    warped by the flow-matching time shift t = a u / (1 + (a - 1) u), a = shift
    (a = 1 keeps the grid uniform; a > 1 spends more steps at high noise).
    The pages give four steps and no values; the warp is the reading taken for
    a non-uniform schedule.  t_S = 0 is implied."""
    if n_steps < 1 or not shift > 0:
        raise ValueError("need n_steps >= 1 and shift > 0")
    out = []
    for s in range(n_steps):
        u = 1.0 - s / n_steps
        out.append(shift * u / (1.0 + (shift - 1.0) * u))
    return tuple(out)


class SlotConflict(RuntimeError):
    pass


class RingPool:
    """Noisy-KV cache: per (stream, block, step) a ring of R slots; chunk c lives
    in slot c mod R.  Each slot records the chunk that wrote it, and a read that
    finds another chunk there raises SlotConflict (a live entry was clobbered)."""

    def __init__(self, n_slots: int):
        self.R = n_slots
        self.slots: Dict[Tuple[int, int, int, int], Tuple[int, np.ndarray, np.ndarray]] = {}

    def write(self, key, chunk, k, v):
        self.slots[key + (chunk % self.R,)] = (chunk, k, v)

    def read(self, key, chunk):
        ent = self.slots.get(key + (chunk % self.R,))
        if ent is None or ent[0] != chunk:
            raise SlotConflict(f"slot of chunk {chunk} at {key} holds {None if ent is None else ent[0]}")
        return ent[1], ent[2]

    def window(self, key, chunk, W):
        """KV of chunks max(0, c - W) .. c - 1, oldest first (fewer when c < W)."""
        return [self.read(key, j) for j in range(max(0, chunk - W), chunk)]


def staggered_ticks(n_chunks: int, n_steps: int, k: int, n_streams: int = 1):
    """Task lists of the staggered schedule: tick tau holds (stream, c, s) with
    c = k (tau - s) + j for 0 <= j < k and 0 <= c < n_chunks."""
    ticks = []
    for tau in range(math.ceil(n_chunks / k) + n_steps - 1):
        tasks = []
        for s in range(n_steps):
            for j in range(k):
                c = k * (tau - s) + j
                if 0 <= c < n_chunks:
                    for sigma in range(n_streams):
                        tasks.append((sigma, c, s))
        ticks.append(tasks)
    return ticks


def _run_batch(tasks, b, w, E, h, pool, contexts_kv, cfg):
    """One block over a batch: all QKV phases and cache writes, then the rest."""
    W, grid, heads = cfg.window, cfg.grid, cfg.heads
    mods, qs = {}, {}
    for (sigma, c, s) in tasks:
        mod = modulation(E[s], w["tmod"])
        q, k, v = qkv_phase(h[(sigma, c)], mod, w, c, grid, heads)
        pool.write((sigma, b, s), c, k, v)
        mods[(sigma, c)], qs[(sigma, c)] = mod, q
    for (sigma, c, s) in tasks:
        ent = pool.window((sigma, b, s), c, W) + [pool.read((sigma, b, s), c)]
        K = np.concatenate([e[0] for e in ent], axis=0)
        V = np.concatenate([e[1] for e in ent], axis=0)
        ck, cv = contexts_kv[(sigma, b)]
        h[(sigma, c)] = rest_phase(h[(sigma, c)], qs[(sigma, c)], K, V, mods[(sigma, c)],
                                   w, ck, cv)


def run_schedule(cfg, blocks: Sequence[dict], tw: dict,
                 latent: Callable[[int, int], np.ndarray],
                 contexts: Sequence[np.ndarray], n_chunks: int,
                 order: str = "sequential", k: int = 1, n_slots: int | None = None,
                 head: dict | None = None):
    """Denoise ``n_chunks`` chunks of each stream through all steps and blocks.

    blocks: weights of blocks 0..B-1; tw: timestep-embedding weights;
    latent(sigma, c): x^0 of a chunk ([L, D] tokens, or [L, P] latent patches
    when ``head`` -- patch embedding and output head weights -- is given);
    contexts[sigma]: conditioning tokens.
    Returns (x_final dict (sigma, c) -> x^S, pool)."""
    S, B = cfg.n_steps, len(blocks)
    ts = list(cfg.timesteps) + [0.0]
    E = [time_embedding(t, tw) for t in cfg.timesteps]
    U = [time_mlp(t, tw) for t in cfg.timesteps] if head is not None else None
    n_streams = len(contexts)
    contexts_kv = {(sg, b): context_kv(contexts[sg], blocks[b], cfg.heads)
                   for sg in range(n_streams) for b in range(B)}
    pool = RingPool(n_slots if n_slots is not None else cfg.window + k)
    x = {(sg, c): np.asarray(latent(sg, c), dtype=F64) for sg in range(n_streams)
         for c in range(n_chunks)}

    if order == "sequential":
        batches = [[[(sg, c, s)]] for sg in range(n_streams) for c in range(n_chunks)
                   for s in range(S)]
        ticks = [b_[0] for b_ in batches]
    elif order == "staggered":
        ticks = staggered_ticks(n_chunks, S, k, n_streams)
    else:
        raise ValueError(order)

    for tasks in ticks:
        if head is None:
            h = {(sg, c): x[(sg, c)].copy() for (sg, c, s) in tasks}
        else:
            h = {(sg, c): patch_embed(x[(sg, c)], head) for (sg, c, s) in tasks}
        for b in range(B):
            _run_batch(tasks, b, blocks[b], E, h, pool, contexts_kv, cfg)
        for (sg, c, s) in tasks:
            v = h[(sg, c)] if head is None else output_head(h[(sg, c)], U[s], head)
            x[(sg, c)] = x[(sg, c)] - (ts[s] - ts[s + 1]) * v
    return x, pool
