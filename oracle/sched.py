"""Multi-stream joint placement of virtual ranks (oracle) -- TEST INFRASTRUCTURE.

What it states (AREX feed article on the PhysisServe report, section "三层设计",
layer 3; 163.com release, section "PhysisServe", bullets "时分复用" and
"虚拟 rank 的动态放置", Fig. 3 and Fig. 4):
  * a stream's per-stage work and state are packed into virtual ranks, and
    virtual ranks are mapped onto physical GPUs; each virtual rank takes one
    memory position of its GPU (Fig. 4);
  * on one GPU, the tasks of the same block are batched -- across chunks,
    steps and streams (Fig. 3 right);
  * a new stream is placed on the GPUs' remaining capacity, by Best-Fit and
    Limited Discrepancy Search; it is admitted only if the whole stream can be
    placed and it meets its SLO running alone; running streams never move.

Readings where the pages are silent (each one a plain choice):
  * stages are (block b, step s) in block-major order p = b * S + s, so that a
    rank holds whole blocks where it can and their steps batch together (as
    one GPU serving one block's four stages); a stream of R virtual ranks takes
    the groups [floor(r N / R), floor((r+1) N / R)); R is the smallest count
    whose every group, alone on a GPU, meets the SLO, or a fixed count;
  * a GPU's cycle -- the time to run every hosted task once, which is the
    chunk interval it sustains -- is sum over blocks of f(n_b), with n_b the
    hosted tasks on block b and f(n) = a + b n for n > 0, f(0) = 0 (one batch
    per block per interval: a fixed part per batch plus a part per task);
  * a placement is feasible when every GPU uses at most M positions and its
    cycle is at most the SLO T;
  * Best-Fit orders the feasible GPUs for a virtual rank by the slack T - cycle
    they would have left, smallest first (ties: lower GPU index); the search
    places the ranks in order r = 0..R-1, and a discrepancy is any choice other
    than the first candidate; LDS with limit D tries limits d = 0..D in turn
    and, at each, depth-first search over paths with at most d discrepancies.

Pinned by ``tests/test_oracle_sched.py``: hand-computed cycles, a small
instance where Best-Fit fails and one discrepancy succeeds, completeness of
LDS with D = R against brute-force enumeration, and invariants.
"""
from __future__ import annotations

import itertools
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple


@dataclass
class Model:
    n_blocks: int          # B
    n_steps: int           # S
    fixed_ms: float        # a: per batch
    per_task_ms: float     # b: per task in a batch

    def f(self, n: int) -> float:
        return 0.0 if n == 0 else self.fixed_ms + self.per_task_ms * n


@dataclass
class Cluster:
    n_gpus: int
    positions: int         # M: virtual ranks per GPU
    slo_ms: float          # T
    model: Model
    n_ranks: int = 0       # virtual ranks per stream (0: the fewest that meet the SLO)
    # per GPU: list of (stream, rank index, {block: task count})
    hosted: List[List[Tuple[int, int, Dict[int, int]]]] = field(default_factory=list)

    def __post_init__(self):
        if not self.hosted:
            self.hosted = [[] for _ in range(self.n_gpus)]


def block_counts(stages: Sequence[Tuple[int, int]]) -> Dict[int, int]:
    out: Dict[int, int] = {}
    for (b, s) in stages:
        out[b] = out.get(b, 0) + 1
    return out


def cycle_ms(model: Model, ranks: Sequence[Dict[int, int]]) -> float:
    """Cycle of a GPU hosting `ranks` (each a {block: tasks} map): one batch
    per block holding every hosted task of that block."""
    tot: Dict[int, int] = {}
    for rk in ranks:
        for b, n in rk.items():
            tot[b] = tot.get(b, 0) + n
    c = 0.0
    for b in sorted(tot):          # block order: a fixed summation order
        c += model.f(tot[b])
    return c


def split_stream(model: Model, slo_ms: float, n_ranks: int = 0) -> Optional[List[Dict[int, int]]]:
    """The stream's virtual ranks: contiguous groups of stages in pipeline
    order, each of which must meet the SLO alone -- the fewest such groups
    (n_ranks = 0) or exactly n_ranks of them; None if that is impossible."""
    B, S = model.n_blocks, model.n_steps
    N = B * S
    stages = [(p // S, p % S) for p in range(N)]     # block-major: all steps of block 0, then block 1, ...
    for R in ([n_ranks] if n_ranks else range(1, N + 1)):
        if R > N:
            return None
        groups = [block_counts(stages[(r * N) // R:((r + 1) * N) // R]) for r in range(R)]
        if all(cycle_ms(model, [g]) <= slo_ms for g in groups):
            return groups
    return None


def _gpu_ranks(cl: Cluster, g: int) -> List[Dict[int, int]]:
    return [rk for (_, _, rk) in cl.hosted[g]]


def candidates(cl: Cluster, rank: Dict[int, int], extra: Dict[int, List[Dict[int, int]]]) -> List[int]:
    """Feasible GPUs for one more virtual rank, in Best-Fit order.  `extra`
    holds the ranks of the stream being placed that are already assigned."""
    out = []
    for g in range(cl.n_gpus):
        ranks = _gpu_ranks(cl, g) + extra.get(g, [])
        if len(ranks) + 1 > cl.positions:
            continue
        c = cycle_ms(cl.model, ranks + [rank])
        if c <= cl.slo_ms:
            out.append((cl.slo_ms - c, g))
    out.sort()
    return [g for (_, g) in out]


def lds_place(cl: Cluster, ranks: Sequence[Dict[int, int]], max_disc: int) -> Optional[List[int]]:
    """GPU of each virtual rank, or None: iterative LDS over limits 0..max_disc."""
    R = len(ranks)

    def dfs(r: int, left: int, extra: Dict[int, List[Dict[int, int]]], chosen: List[int]):
        if r == R:
            return list(chosen)
        for i, g in enumerate(candidates(cl, ranks[r], extra)):
            cost = 0 if i == 0 else 1
            if cost > left:
                break
            extra.setdefault(g, []).append(ranks[r])
            chosen.append(g)
            got = dfs(r + 1, left - cost, extra, chosen)
            chosen.pop()
            extra[g].pop()
            if got is not None:
                return got
        return None

    for d in range(max_disc + 1):
        got = dfs(0, d, {}, [])
        if got is not None:
            return got
    return None


def admit(cl: Cluster, stream: int, max_disc: int) -> Optional[List[int]]:
    """Admits `stream` if it meets the SLO alone and all its virtual ranks can
    be placed; running streams stay where they are.  Returns the GPUs of its
    ranks, or None (cluster unchanged)."""
    ranks = split_stream(cl.model, cl.slo_ms, cl.n_ranks)
    if ranks is None:
        return None
    place = lds_place(cl, ranks, max_disc)
    if place is None:
        return None
    for r, g in enumerate(place):
        cl.hosted[g].append((stream, r, ranks[r]))
    return place


def release(cl: Cluster, stream: int) -> int:
    """Removes a stream's virtual ranks; returns how many there were."""
    n = 0
    for g in range(cl.n_gpus):
        keep = [e for e in cl.hosted[g] if e[0] != stream]
        n += len(cl.hosted[g]) - len(keep)
        cl.hosted[g] = keep
    return n


def feasible(cl: Cluster) -> bool:
    return all(len(cl.hosted[g]) <= cl.positions and cycle_ms(cl.model, _gpu_ranks(cl, g)) <= cl.slo_ms
               for g in range(cl.n_gpus))


def exists_placement(cl: Cluster, ranks: Sequence[Dict[int, int]]) -> bool:
    """Brute force: is there any assignment of `ranks` to GPUs that keeps the
    cluster feasible?  (Small instances only.)"""
    for assign in itertools.product(range(cl.n_gpus), repeat=len(ranks)):
        ok = True
        for g in range(cl.n_gpus):
            mine = [ranks[r] for r in range(len(ranks)) if assign[r] == g]
            if not mine:
                continue
            allr = _gpu_ranks(cl, g) + mine
            if len(allr) > cl.positions or cycle_ms(cl.model, allr) > cl.slo_ms:
                ok = False
                break
        if ok:
            return True
    return False


def equal_split_streams(n_gpus: int, model: Model, slo_ms: float) -> int:
    """Streams served when each gets its own group of GPUs, one virtual rank
    per GPU (no sharing, no cross-stream batching): floor(G / R), R the fewest
    ranks that meet the SLO."""
    ranks = split_stream(model, slo_ms)
    return 0 if ranks is None else n_gpus // len(ranks)
