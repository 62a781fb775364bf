"""Host logic of the placed-stage runner (no GPU): which tasks each block batch
of each tick holds, against the stage pipeline's definition and its
dependencies."""
import json
import os

import pytest

from autoregressive_denoising_dit_amd.runner import model_cycle_ms, n_ticks, rank_stages, tick_tasks

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _simulate(B, S, n_chunks, starts, hosted=None):
    N = B * S
    hosted = hosted or {sg: list(range(N)) for sg in starts}
    when = {}
    batches = []
    for tau in range(n_ticks(starts, B, S, n_chunks)):
        for b in reversed(range(B)):
            tl = tick_tasks(tau, b, hosted, starts, B, S, n_chunks)
            batches.append((tau, b, tl))
            for (sg, s, c) in tl:
                assert (sg, c, s, b) not in when
                when[(sg, c, s, b)] = tau
    return when, batches


def test_fig2_stage_path_one_block_per_tick():
    """The release's 2-step x 4-block example: chunk 7 passes the 8 stages in
    step-major order, one stage per tick, and once the pipeline is full one
    chunk leaves it per tick."""
    g = json.load(open(os.path.join(GOLDEN, "fig2_stage_pipeline.json")))
    S, B, c7 = g["n_steps"], g["n_blocks"], g["chunk"]
    when, _ = _simulate(B, S, 12, {0: 0})
    path = sorted(((t, s, b) for (sg, c, s, b), t in when.items() if c == c7))
    assert [[s, b] for (_, s, b) in path] == g["stage_path_of_chunk"]
    assert [t for (t, _, _) in path] == list(range(path[0][0], path[0][0] + S * B))
    done = {}
    for (sg, c, s, b), t in when.items():
        if s == S - 1 and b == B - 1:
            done[t] = done.get(t, 0) + 1
    fill = S * B - 1
    assert all(done.get(t, 0) == g["completions_per_interval_after_fill"] for t in range(fill, fill + 12))


@pytest.mark.parametrize("B,S,W,starts", [(2, 2, 2, {0: 0, 1: 1, 2: 3}), (3, 4, 3, {0: 0, 5: 2}), (1, 3, 1, {0: 4})])
def test_every_task_once_and_dependencies_hold(B, S, W, starts):
    n_chunks = 6
    when, batches = _simulate(B, S, n_chunks, starts)
    assert len(when) == len(starts) * n_chunks * S * B
    for (sg, c, s, b), t in when.items():
        assert t == starts[sg] + c + s * B + b                      # the pipeline position
        if b > 0:
            assert when[(sg, c, s, b - 1)] == t - 1                 # hidden state from the previous block
        elif s > 0:
            assert when[(sg, c, s - 1, B - 1)] == t - 1             # latent after the previous step's Euler
        for j in range(max(0, c - W), c):
            assert when[(sg, j, s, b)] < t                          # noisy KV written in an earlier tick
        # ring of W + 1 slots: the chunk that last used this slot has no reader left
        if c >= W + 1:
            last_reader = c - 1
            assert when[(sg, last_reader, s, b)] < t
    # a batch never holds two tasks of one (stream, step)
    for tau, b, tl in batches:
        assert len({(sg, s) for (sg, s, c) in tl}) == len(tl)


def test_steady_state_batches_hold_every_step_of_every_stream():
    B, S = 3, 4
    starts = {0: 0, 1: 2, 2: 5}
    _, batches = _simulate(B, S, 20, starts)
    steady = [len(tl) for (tau, b, tl) in batches if 5 + S * B <= tau < 20]
    assert steady and all(n == S * len(starts) for n in steady)


def test_partial_hosting_selects_the_hosted_stages():
    B, S = 2, 3
    hosted = {0: [p for p in range(B * S) if p // S == 1]}      # block 1 only
    _, batches = _simulate(B, S, 4, {0: 0}, hosted=hosted)
    assert all(tl == [] for (tau, b, tl) in batches if b == 0)
    assert any(tl for (tau, b, tl) in batches if b == 1)


@pytest.mark.parametrize("N,R", [(8, 1), (8, 3), (120, 7), (5, 5)])
def test_rank_stages_partition(N, R):
    spans = [rank_stages(N, R, r) for r in range(R)]
    assert spans[0][0] == 0 and spans[-1][1] == N
    for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
        assert a1 == b0 and a0 < a1


@pytest.mark.parametrize("B,S,R", [(30, 4, 1), (30, 4, 7), (2, 2, 3), (5, 3, 15)])
def test_ranks_and_cycle_match_the_placement_model(B, S, R):
    """The runner's rank split and its cost of a full tick are the placement
    oracle's: the same block composition per rank, the same a + b n sum."""
    from oracle import sched as osched
    model = osched.Model(B, S, 0.279, 0.199)
    groups = osched.split_stream(model, 1e9, n_ranks=R)
    N = B * S
    for r in range(R):
        p0, p1 = rank_stages(N, R, r)
        mine = {}
        for p in range(p0, p1):
            mine[p // S] = mine.get(p // S, 0) + 1
        assert mine == groups[r]
    hosted = {0: list(range(N)), 3: list(range(*rank_stages(N, R, 0)))}
    ranks = groups + [groups[0]]
    assert model_cycle_ms(hosted, S, 0.279, 0.199) == pytest.approx(osched.cycle_ms(model, ranks), rel=1e-12)
