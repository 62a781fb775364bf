"""The placed-stage runner on the GPU: the virtual ranks that the joint
placement assigns to one GPU, run as the stage pipeline with one batch per
block per tick, against the oracle's sequential schedule."""
import numpy as np
import pytest
import torch

import oracle
from autoregressive_denoising_dit_amd.runner import PlacedRunner, rank_stages
from autoregressive_denoising_dit_amd.sched import Scheduler
from synthetic import C1, inputs, with_
from tests.gpu_util import host, make_block, make_pool, make_te, rel_err, say, to_dev, tol

pytestmark = pytest.mark.gpu


def _placed(cfg, streams, starts, n_chunks, ranks_per_stream):
    B, S, W = cfg.n_blocks, cfg.n_steps, cfg.window
    sched = Scheduler(1, 4 * ranks_per_stream * len(streams), B, S, 1e6, 0.1, 0.1, 1, ranks_per_stream)
    ranks = []
    for sg in streams:
        gpus = sched.admit(sg)
        assert gpus == [0] * ranks_per_stream, gpus
        ranks += [(sg, *rank_stages(B * S, ranks_per_stream, r)) for r in range(ranks_per_stream)]
    blocks = [inputs.block_weights(cfg, b, 0) for b in range(B)]
    tw = inputs.time_weights(cfg, 0)
    ctxs = {sg: inputs.context(cfg, sg, 0) for sg in streams}
    lat = {(sg, c): inputs.latent(cfg, sg, c, 0) for sg in streams for c in range(n_chunks)}
    td = torch.float32 if cfg.dtype == "fp32" else torch.bfloat16
    pool = make_pool(cfg, n_streams=max(streams) + 1, n_blocks=B, n_slots=W + 1)
    blks = [make_block(cfg, w, b) for b, w in enumerate(blocks)]
    te = make_te(cfg, tw)
    for blk in blks:
        for sg in streams:
            pool.context_set(blk, sg, to_dev(ctxs[sg], td))
    x = {sg: torch.stack([to_dev(lat[(sg, c)], torch.float32) for c in range(n_chunks)]).contiguous()
         for sg in streams}
    runner = PlacedRunner(pool, blks, te, cfg.timesteps, W, ranks, starts, n_chunks)
    sizes = []
    runner.run(x, on_tick=lambda tau, s: sizes.append(list(s)))
    torch.cuda.synchronize()
    # the oracle's streams are numbered 0..; map them
    order = sorted(streams)
    ox, _ = oracle.run_schedule(cfg, blocks, tw, lambda i, c: lat[(order[i], c)], [ctxs[sg] for sg in order],
                                n_chunks, order="sequential")
    return {sg: host(x[sg]) for sg in streams}, {(order[i], c): v for (i, c), v in ox.items()}, lat, sizes


def test_placed_runner_c1_three_streams_offset_phases():
    """Three streams started at ticks 0, 1 and 3 (offset phases), each split
    into two virtual ranks that the placement puts on the one GPU; every
    chunk's x^S against the sequential oracle at the fp32 bound."""
    cfg = C1
    streams, starts, n_chunks = [0, 1, 2], {0: 0, 1: 1, 2: 3}, 6
    say("placed runner c1, streams", streams, "starts", starts)
    gx, ox, _, sizes = _placed(cfg, streams, starts, n_chunks, ranks_per_stream=2)
    # batches mixed steps and streams at offset phases
    assert max(max(s) for s in sizes) == len(streams) * cfg.n_steps
    assert any(0 < n < len(streams) * cfg.n_steps for s in sizes for n in s)
    for sg in streams:
        for c in range(n_chunks):
            e = rel_err(gx[sg][c], ox[(sg, c)])
            say(f"stream {sg} chunk {c}: x^S err {e:.2e}")
            assert e <= tol(cfg)


def test_placed_runner_bf16_small_width():
    """The same at bf16 with 64-dim heads and full-length chunks (two streams,
    one virtual rank each, 2 blocks x 2 steps)."""
    cfg = with_(C1, dtype="bf16", hidden=256, heads=4, head_dim=64, ffn=512, grid=(1, 12, 16), n_ctx=32)
    streams, starts, n_chunks = [1, 4], {1: 0, 4: 2}, 3
    say("placed runner bf16, streams", streams, "starts", starts)
    gx, ox, _, _ = _placed(cfg, streams, starts, n_chunks, ranks_per_stream=1)
    for sg in streams:
        for c in range(n_chunks):
            e = rel_err(gx[sg][c], ox[(sg, c)])
            say(f"stream {sg} chunk {c}: x^S err {e:.2e}")
            assert e <= tol(cfg)
