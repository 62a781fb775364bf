"""Host driver of the staggered chunk x step schedule on one GPU.

Each chunk starts from noise and passes S denoising steps; chunk c + 1 does not
wait for chunk c to finish -- it reads the noisy KV chunk c left at the same
step, so adjacent chunks' denoising is offset and overlaps (AREX feed article
on the PhysisServe report, section "难题"; 163.com release, section
"新一代物理 AI 的基础设施", Fig. 1).  One GPU time-shares all stages and, per
block, batches the tasks of different chunks and steps (AREX article,
"三层设计", layer 2; 163.com release, bullet "时分复用").

Tick tau holds the tasks (stream, c, s) with c = k (tau - s) + j, 0 <= j < k.
For each block b the tick's tasks form one ps_stage_batch call; after the last
block every task takes its Euler step.  Tasks are ordered by chunk, then
stream, so that with latents stored chunk-major the tick's rows are one
contiguous slice: the first block reads the latents in place and the Euler
step updates them in place -- no gather or scatter copies.

Ring slots: chunk c uses slot c mod R of its (stream, block, step), R >= W + k;
it reads the slots of chunks max(0, c - W) .. c - 1 (fewer while c < W).

With a patch embedding and output head (``runtime.Head``) the latents are a
chunk's latent patches [L, P]: the tick's rows are embedded into the residual
stream before block 0, and after the last block the head turns each task's
rows into the velocity of its Euler step.
"""
from __future__ import annotations

import math
from typing import Callable, List, Optional, Sequence, Tuple

import torch

from . import runtime
from .runtime import Block, Head, Pool, TimeEmbed


def shifted_timesteps(n_steps: int, shift: float = 1.0) -> Tuple[float, ...]:
    """Timesteps t_0 > ... > t_{S-1} (t_S = 0): the uniform grid u = 1 - s/S
    under the flow-matching time shift t = a u / (1 + (a - 1) u), a = shift,
    computed by the library (ps_timesteps).  a = 1 is the uniform schedule;
    a > 1 spends more of the steps at high noise.  The pages fix four steps
    but no values."""
    if n_steps < 1 or not shift > 0:
        raise ValueError("need n_steps >= 1 and shift > 0")
    return tuple(runtime.timesteps(n_steps, shift))


def tick_tasks(tau: int, n_chunks: int, n_steps: int, k: int, n_streams: int) -> List[Tuple[int, int, int]]:
    """(stream, chunk, step) of tick tau, ordered by chunk then stream."""
    out = []
    for s in range(n_steps - 1, -1, -1):          # older chunks (later steps) first
        for j in range(k):
            c = k * (tau - s) + j
            if 0 <= c < n_chunks:
                for sg in range(n_streams):
                    out.append((sg, c, s))
    out.sort(key=lambda t: (t[1], t[0]))
    return out


def n_ticks(n_chunks: int, n_steps: int, k: int) -> int:
    return math.ceil(n_chunks / k) + n_steps - 1


class StaggeredRunner:
    """Runs the staggered schedule of `n_chunks` chunks of `n_streams` streams.

    groups > 1 splits each tick's tasks into that many groups of consecutive
    steps (the tick's task list is ordered by chunk, so each group is a
    contiguous slice of the latents).  The groups share no dependency inside a
    tick -- a task reads the noisy KV of its own step and its own hidden state
    -- so their block batches run concurrently on separate HIP streams, one
    group's partial rounds of tiles overlapping the other's work; the tick ends
    when every group has finished.  A task's results do not depend on its batch
    companions, so the grouping changes no result."""

    def __init__(self, pool: Pool, blocks: Sequence[Block], te: TimeEmbed, timesteps: Sequence[float],
                 window: int, k: int, n_streams: int, head: Optional[Head] = None, groups: int = 1):
        if pool.n_slots < window + k:
            raise ValueError(f"ring of {pool.n_slots} slots is smaller than window + k = {window + k}")
        if head is not None and head.hidden != pool.hidden:
            raise ValueError("head width differs from the pool's")
        self.pool, self.blocks, self.te, self.head = pool, list(blocks), te, head
        self.ts = list(timesteps) + [0.0]
        self.S, self.W, self.k, self.n_streams = len(timesteps), window, k, n_streams
        self.L, self.D = pool.tokens, pool.hidden
        self.P = head.latent_dim if head is not None else self.D   # latent values per token
        rows = self.S * k * n_streams * self.L
        self.hbuf = torch.empty((rows, self.D), dtype=torch.float32, device="cuda")
        self.vbuf = torch.empty((rows, self.P), dtype=torch.float32, device="cuda") if head is not None else None
        if not 1 <= groups <= min(self.S, 4):
            raise ValueError(f"groups must be in [1, {min(self.S, 4)}]")
        if groups > 1 and head is not None:
            raise ValueError("the head's workspace serves one stream: groups > 1 needs head=None")
        self.groups = groups
        self.side = [torch.cuda.Stream() for _ in range(groups - 1)]

    def tasks_for(self, tau: int, n_chunks: int):
        tl = tick_tasks(tau, n_chunks, self.S, self.k, self.n_streams)
        R = self.pool.n_slots
        ps_tasks = []
        for (sg, c, s) in tl:
            nr = min(self.W, c)
            ps_tasks.append(runtime.make_task(sg, c, s, self.ts[s], c % R,
                                              [(c - nr + i) % R for i in range(nr)]))
        return tl, ps_tasks

    def _run_group(self, tl, tasks, x, row0, cuda_stream):
        """All blocks, then the head and Euler, for one group of the tick's
        tasks (rows row0 .. of the tick's slice)."""
        c_lo = tl[0][1]
        n = len(tl)
        rows = n * self.L
        xs = x[c_lo:c_lo + n // self.n_streams].view(rows, self.P)
        h = self.hbuf[row0:row0 + rows]
        if self.head is not None:
            runtime.patch_embed(self.head, xs, h, cuda_stream=cuda_stream)
        for b, blk in enumerate(self.blocks):
            runtime.stage_batch(self.pool, blk, self.te, tasks, xs if (b == 0 and self.head is None) else h, h,
                                cuda_stream=cuda_stream)
        steps = [s for (_, _, s) in tl]
        if self.head is not None:
            v = self.vbuf[row0:row0 + rows]
            runtime.output_head(self.head, self.te, [self.ts[s] for s in steps], self.L, h, v, cuda_stream=cuda_stream)
            runtime.euler_update_steps(xs, v, self.ts[:-1], steps, self.L, self.P, cuda_stream=cuda_stream)
        else:
            runtime.euler_update_steps(xs, h, self.ts[:-1], steps, self.L, self.D, cuda_stream=cuda_stream)

    def run_tick(self, tau: int, x: torch.Tensor, n_chunks: int):
        """x: fp32 [n_chunks, n_streams, L, P] latents (P = D without a head),
        updated in place."""
        tl, tasks = self.tasks_for(tau, n_chunks)
        if not tl:
            return tl
        if self.groups == 1:
            self._run_group(tl, tasks, x, 0, None)
            return tl
        # split by step into groups of whole steps (each a run of consecutive
        # chunks); group 0 on the current stream, the others on side streams
        steps = sorted({s for (_, _, s) in tl}, reverse=True)
        per = -(-len(steps) // self.groups)
        parts = [set(steps[i:i + per]) for i in range(0, len(steps), per)]
        main = torch.cuda.current_stream()
        start = torch.cuda.Event()
        start.record(main)
        row0 = 0
        for gi, part in enumerate(parts):
            idx = [i for i, t in enumerate(tl) if t[2] in part]
            sub_tl, sub_tasks = [tl[i] for i in idx], [tasks[i] for i in idx]
            st = main if gi == 0 else self.side[gi - 1]
            if gi > 0:
                st.wait_event(start)
            self._run_group(sub_tl, sub_tasks, x, row0, None if gi == 0 else st)
            row0 += len(idx) * self.L
        for st in self.side[:len(parts) - 1]:
            done = torch.cuda.Event()
            done.record(st)
            main.wait_event(done)
        return tl

    def run(self, x: torch.Tensor, n_chunks: int, on_tick: Optional[Callable[[int, list], None]] = None):
        for tau in range(n_ticks(n_chunks, self.S, self.k)):
            tl = self.run_tick(tau, x, n_chunks)
            if on_tick is not None:
                on_tick(tau, tl)
