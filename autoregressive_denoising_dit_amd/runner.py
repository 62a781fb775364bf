"""Host driver of the stage groups that the joint placement puts on one GPU.

A stream's stages (block b, step s) are grouped into virtual ranks in
block-major order p = b * S + s; the placement maps each rank to a GPU
(``sched.Scheduler``; AREX feed article on the PhysisServe report, section
"三层设计", layer 3; 163.com release, bullet "虚拟 rank 的动态放置", Fig. 4).
This runner executes the ranks hosted by one GPU as the pages' stage
pipeline (163.com release, bullet "Stage-wise 流水线", Fig. 2): chunk c of
stream sigma is at stage (s, b) -- path position j = s * B + b -- at tick
start[sigma] + c + j, so every stage takes one chunk per tick and a stream
completes one chunk per tick once its pipeline is full.  In each tick the GPU
time-shares its stages (same release, bullet "时分复用", Fig. 3 right): for
each block it runs one batch of whichever hosted tasks of that block are
ready, across steps and streams whose phases differ.

The tasks of one tick are independent: stage (s, b) reads the hidden state
stage (s, b - 1) left in the previous tick and the noisy KV of earlier chunks
at (b, s), written in earlier ticks.  Blocks run in descending order within a
tick, so that a stage's hand-off buffer is read by the next block's batch
before this block's batch overwrites it.  After the last block, each task's
chunk takes its Euler step; the next step's first block reads that latent in a
later tick.  Ring slots: chunk c uses slot c mod R, R >= W + 1.

Only streams whose stages are all hosted here run end to end (the hand-off of
hidden states between GPUs is not part of this single-GPU build).
"""
from __future__ import annotations

from typing import Callable, Dict, List, Optional, Sequence, Tuple

import torch

from . import runtime
from .runtime import Block, Pool, TimeEmbed


def rank_stages(n_stages: int, n_ranks: int, r: int) -> Tuple[int, int]:
    """Stages [p0, p1) of virtual rank r of a stream split into n_ranks groups
    (the placement's split: floor(r N / R) .. floor((r + 1) N / R))."""
    return (r * n_stages) // n_ranks, ((r + 1) * n_stages) // n_ranks


def tick_tasks(tau: int, b: int, hosted: Dict[int, Sequence[int]], starts: Dict[int, int], n_blocks: int,
               n_steps: int, n_chunks: int) -> List[Tuple[int, int, int]]:
    """(stream, step, chunk) of the hosted tasks of block b ready at tick tau,
    ordered by stream then step.  hosted[sigma]: the stages p = b * S + s of
    stream sigma on this GPU."""
    out = []
    for sg in sorted(hosted):
        for p in sorted(hosted[sg]):
            bp, s = divmod(p, n_steps)
            if bp != b:
                continue
            c = tau - starts[sg] - (s * n_blocks + b)
            if 0 <= c < n_chunks:
                out.append((sg, s, c))
    return out


def model_cycle_ms(hosted: Dict[int, Sequence[int]], n_steps: int, batch_fixed_ms: float,
                   batch_task_ms: float) -> float:
    """The placement's cost of one full tick of a GPU hosting these stages:
    the sum over blocks (in block order) of a + b n_b, n_b the hosted tasks of
    block b (one per hosted stage of that block)."""
    per_block: Dict[int, int] = {}
    for ps in hosted.values():
        for p in ps:
            per_block[p // n_steps] = per_block.get(p // n_steps, 0) + 1
    c = 0.0
    for b in sorted(per_block):
        c += batch_fixed_ms + batch_task_ms * per_block[b]
    return c


def n_ticks(starts: Dict[int, int], n_blocks: int, n_steps: int, n_chunks: int) -> int:
    """Ticks until the last chunk of every stream has left the pipeline."""
    return max(starts.values()) + n_chunks + n_blocks * n_steps - 1


class PlacedRunner:
    """Runs the virtual ranks hosted on this GPU.

    ranks: (stream, p0, p1) for every hosted rank; starts[stream]: the tick at
    which the stream's chunk 0 enters stage (0, 0)."""

    def __init__(self, pool: Pool, blocks: Sequence[Block], te: TimeEmbed, timesteps: Sequence[float], window: int,
                 ranks: Sequence[Tuple[int, int, int]], starts: Dict[int, int], n_chunks: int):
        self.pool, self.blocks, self.te = pool, list(blocks), te
        self.ts = list(timesteps)
        self.S, self.B, self.W = len(timesteps), len(blocks), window
        if pool.n_slots < window + 1:
            raise ValueError(f"ring of {pool.n_slots} slots is smaller than window + 1 = {window + 1}")
        N = self.B * self.S
        self.hosted: Dict[int, List[int]] = {}
        for (sg, p0, p1) in ranks:
            if not 0 <= p0 < p1 <= N:
                raise ValueError(f"rank ({sg}, {p0}, {p1}) outside stages 0..{N}")
            self.hosted.setdefault(sg, []).extend(range(p0, p1))
        for sg, ps in self.hosted.items():
            if sorted(ps) != list(range(N)):
                raise ValueError(f"stream {sg}: its stages are not all hosted here exactly once")
            if sg not in starts:
                raise ValueError(f"stream {sg}: no start tick")
        self.starts, self.n_chunks = dict(starts), n_chunks
        self.L, self.D = pool.tokens, pool.hidden
        # hand-off buffers: the hidden state each stage (path position j) left
        self.h = {sg: torch.empty((N, self.L, self.D), dtype=torch.float32, device="cuda") for sg in self.hosted}
        self.tick_blocks: List[int] = []   # tasks per block batch of the last tick

    def n_ticks(self) -> int:
        return n_ticks(self.starts, self.B, self.S, self.n_chunks)

    def run_tick(self, tau: int, x: Dict[int, torch.Tensor]) -> List[int]:
        """x[stream]: fp32 [n_chunks, L, D] latents, updated in place.  Returns
        the batch size of each block (0 where no task was ready)."""
        R = self.pool.n_slots
        sizes = [0] * self.B
        for b in reversed(range(self.B)):
            tl = tick_tasks(tau, b, self.hosted, self.starts, self.B, self.S, self.n_chunks)
            if not tl:
                continue
            sizes[b] = len(tl)
            tasks, h_in, h_out = [], [], []
            for (sg, s, c) in tl:
                nr = min(self.W, c)
                tasks.append(runtime.make_task(sg, c, s, self.ts[s], c % R, [(c - nr + i) % R for i in range(nr)]))
                j = s * self.B + b
                h_in.append(x[sg][c] if b == 0 else self.h[sg][j - 1])
                h_out.append(self.h[sg][j])
            runtime.stage_batch_rows(self.pool, self.blocks[b], self.te, tasks, h_in, h_out)
            if b == self.B - 1:
                for (sg, s, c) in tl:
                    runtime.euler_update_steps(x[sg][c], self.h[sg][s * self.B + b], self.ts, [s], self.L, self.D)
        self.tick_blocks = sizes
        return sizes

    def run(self, x: Dict[int, torch.Tensor], on_tick: Optional[Callable[[int, List[int]], None]] = None):
        for tau in range(self.n_ticks()):
            sizes = self.run_tick(tau, x)
            if on_tick is not None:
                on_tick(tau, sizes)

    def model_cycle_ms(self, batch_fixed_ms: float, batch_task_ms: float) -> float:
        return model_cycle_ms(self.hosted, self.S, batch_fixed_ms, batch_task_ms)
