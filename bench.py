#!/usr/bin/env python3
"""Stage-task throughput on one MI355X (gfx950).

A step is one pass of the whole stage path over one batch of synthetic input:
batch formation, per-task modulation, AdaLN + QKV + 3D RoPE + cache write,
self-attention over the noisy-KV window, gated O projection, cross-attention,
the gated GELU-tanh FFN, and the flow-matching Euler update of the batch's
latents.  Default workload: the Wan2.1-14B-shaped stage, 16 tasks from 16
streams at mixed denoising steps per batch (hidden 5120, 40 x 128 heads, FFN
13824, 1560 tokens per chunk, window of 3 prior chunks, 512 conditioning
tokens, bf16 operands).  Weights are random-init of that shape (no trained
weights are available), inputs seeded, everything resident in HBM before the
timed region starts.

Prints one JSON line: stage tasks/s, ms per step, the steady-state chunk
interval, the fraction of the bf16 MFMA peak, a roofline record of the
dominant kernel and the CPU oracle timed on a bounded sample of the same
workload.  The timed steps run without per-kernel events; the same number of
steps then runs again with a HIP event pair around every kernel (recorded by
the library on the kernel's stream), which gives the per-kernel durations and
the roofline record's.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

PEAK = {"bf16": 2516.6e12, "fp32": 157.3e12}   # dense MFMA, 256 CU x 2.4 GHz
MI355X_XCDS, MI355X_SIMDS = 8, 256 * 4          # accelerator dies, SIMDs (4 per CU)
HBM_PEAK = 8.0e12


def _log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_work(cfg, n_tasks, n_read):
    """Algorithmic FLOPs (contractions) or bytes (memory-bound kernels) per launch."""
    L, D, F, Lc = cfg.tokens, cfg.hidden, cfg.ffn, cfg.n_ctx
    M = n_tasks * L
    es = 2 if cfg.dtype == "bf16" else 4
    return {
        "qkv": ("flop", 2 * M * D * 3 * D),
        "attn_self": ("flop", 4 * L * (n_read + 1) * L * D * n_tasks),
        "o_proj": ("flop", 2 * M * D * D),
        "xq_proj": ("flop", 2 * M * D * D),
        "attn_cross": ("flop", 4 * L * Lc * D * n_tasks),
        "xo_proj": ("flop", 2 * M * D * D),
        "ffn1": ("flop", 2 * M * D * F),
        "ffn2": ("flop", 2 * M * F * D),
        "ln1": ("byte", M * D * (4 + es)),
        "ln2": ("byte", M * D * (4 + es)),
        "ln3": ("byte", M * D * (4 + es)),
        "euler": ("byte", M * D * 12),
    }


def cache_bytes(cfg, n_tasks, n_read):
    """Cached keys and values an attention launch reads (algorithmic bytes):
    the window's noisy KV for self-attention, the context K/V for cross."""
    es = 2 if cfg.dtype == "bf16" else 4
    return {"attn_self": n_tasks * (n_read + 1) * cfg.tokens * cfg.hidden * 2 * es,
            "attn_cross": n_tasks * cfg.n_ctx * cfg.hidden * 2 * es}


def setup_stage(cfg, n_tasks, seed=0):
    """Device-resident weights, pool, contexts and inputs for single-stage runs."""
    import torch
    from autoregressive_denoising_dit_amd import runtime
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    td = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    D, F, H, d = cfg.hidden, cfg.ffn, cfg.heads, cfg.head_dim

    def rn(*shape, dtype=torch.float32, std=0.02):
        return (torch.randn(*shape, generator=g, device="cuda") * std).to(dtype).contiguous()

    w = {"wqkv": rn(3 * D, D, dtype=td), "wo": rn(D, D, dtype=td), "wq2": rn(D, D, dtype=td),
         "wkv2": rn(2 * D, D, dtype=td), "wo2": rn(D, D, dtype=td), "w1": rn(F, D, dtype=td),
         "w2": rn(D, F, dtype=td), "bqkv": rn(3 * D), "bo": rn(D), "bq2": rn(D), "bkv2": rn(2 * D),
         "bo2": rn(D), "b1": rn(F), "b2": rn(D), "tmod": rn(6, D)}
    tw = {"wt1": rn(D, 256), "bt1": rn(D), "wt2": rn(D, D), "bt2": rn(D), "wp": rn(6 * D, D), "bp": rn(6 * D)}
    n_streams = n_tasks
    R = cfg.window + 1
    pool = runtime.Pool(n_streams, 1, cfg.n_steps, R, cfg.grid, H, d, cfg.n_ctx, runtime.ps_dtype(cfg.dtype))
    blk = runtime.Block(w, D, H, d, F, 0, runtime.ps_dtype(cfg.dtype))
    te = runtime.TimeEmbed(tw, D, capacity=16)
    kv_k = rn(cfg.tokens, H, d, dtype=td, std=1.0)
    kv_v = rn(cfg.tokens, H, d, dtype=td, std=1.0)
    for sg in range(n_streams):
        pool.context_set(blk, sg, rn(cfg.n_ctx, D, dtype=td, std=1.0))
        for s in range(cfg.n_steps):
            for slot in range(R):
                pool.load(sg, 0, s, slot, 0, kv_k, kv_v)
    x = rn(n_tasks * cfg.tokens, D, std=1.0)
    h = torch.empty_like(x)
    xe = x.clone()
    torch.cuda.synchronize()
    return dict(pool=pool, blk=blk, te=te, x=x, h=h, xe=xe, w=w, tw=tw)


def run_stagger_bench(cfg, measured=64, with_head=False, groups=1):
    """Steady-state chunk interval of one stream under the staggered schedule
    (all blocks, all steps, k chunks per step per tick): `measured` chunks
    completed after a warm-up of S + W + 2 ticks, from events recorded after
    each tick's Euler step.  As many further ticks then run with per-kernel
    events, for the time per tick of each kernel.  With `with_head` the
    latents are latent patches [L, P]: the patch embedding runs before block 0
    and the output head after the last block of every tick."""
    import torch
    from autoregressive_denoising_dit_amd import runtime
    from autoregressive_denoising_dit_amd.schedule import StaggeredRunner
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    td = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    D, F, H, d, B, S, W, k = cfg.hidden, cfg.ffn, cfg.heads, cfg.head_dim, cfg.n_blocks, cfg.n_steps, cfg.window, cfg.k

    def rn(*shape, dtype=torch.float32, std=0.02):
        return (torch.randn(*shape, generator=g, device="cuda") * std).to(dtype).contiguous()

    _log(f"setting up {cfg.name}: {B} blocks x {S} steps, k = {k}")
    blocks, keep = [], []
    pool = runtime.Pool(1, B, S, W + k, cfg.grid, H, d, cfg.n_ctx, runtime.ps_dtype(cfg.dtype))
    for b in range(B):
        w = {"wqkv": rn(3 * D, D, dtype=td), "wo": rn(D, D, dtype=td), "wq2": rn(D, D, dtype=td),
             "wkv2": rn(2 * D, D, dtype=td), "wo2": rn(D, D, dtype=td), "w1": rn(F, D, dtype=td),
             "w2": rn(D, F, dtype=td), "bqkv": rn(3 * D), "bo": rn(D), "bq2": rn(D), "bkv2": rn(2 * D),
             "bo2": rn(D), "b1": rn(F), "b2": rn(D), "tmod": rn(6, D)}
        blk = runtime.Block(w, D, H, d, F, b, runtime.ps_dtype(cfg.dtype))
        pool.context_set(blk, 0, rn(cfg.n_ctx, D, dtype=td, std=1.0))
        blocks.append(blk)
        keep.append(w)
    tw = {"wt1": rn(D, 256), "bt1": rn(D), "wt2": rn(D, D), "bt2": rn(D), "wp": rn(6 * D, D), "bp": rn(6 * D)}
    te = runtime.TimeEmbed(tw, D, capacity=16)
    head = None
    if with_head:
        P = cfg.latent_dim
        head = runtime.Head({"w_embed": rn(D, P, dtype=td), "w_head": rn(P, D, dtype=td), "b_embed": rn(D),
                             "b_head": rn(P), "t_head": rn(2, D)}, D, P, runtime.ps_dtype(cfg.dtype))
    runner = StaggeredRunner(pool, blocks, te, cfg.timesteps, W, k, 1, head=head, groups=groups)
    tau0 = S + W + 2                       # warm-up ticks (pipeline filled, full windows)
    tau1 = tau0 + (measured + k - 1) // k  # each later tick completes k chunks
    tau2 = tau1 + (tau1 - tau0)            # then as many ticks again with per-kernel events
    n_chunks = k * (tau2 + 1)
    x = rn(n_chunks, 1, cfg.tokens, cfg.latent_dim if with_head else D, std=1.0)
    from autoregressive_denoising_dit_amd import _lib
    torch.cuda.synchronize()
    ev = {}
    for tau in range(tau2 + 1):
        if tau == tau1 + 1:
            torch.cuda.synchronize()
            _lib.trace_enable(True)
        runner.run_tick(tau, x, n_chunks)
        if tau0 <= tau <= tau1:
            ev[tau] = torch.cuda.Event(enable_timing=True)
            ev[tau].record()
    torch.cuda.synchronize()
    trace = _lib.trace_read()
    _lib.trace_enable(False)
    assert torch.isfinite(x).all().item(), "non-finite latents"
    done = k * (tau1 - tau0)
    interval = ev[tau0].elapsed_time(ev[tau1]) / done
    tick = ev[tau0].elapsed_time(ev[tau1]) / (tau1 - tau0)
    per_tick = {n: round(ms / (tau2 - tau1), 3) for n, (_, ms) in trace.items()}
    return interval, tick, done, per_tick


def run_batch_sweep(cfg, sizes=(1, 2, 4, 8, 16), steps=20, warmup=4):
    """Time of one block batch (ps_stage_batch, full windows, steps mixed) for
    each batch size n; least-squares fit t(n) = a + b n."""
    import numpy as np
    import torch
    from autoregressive_denoising_dit_amd import runtime
    out = {}
    for n in sizes:
        _log(f"batch sweep {cfg.name}: {n} tasks")
        st = setup_stage(cfg, n)
        tls = [stage_tasks(cfg, n, tau) for tau in range(cfg.n_steps)]
        for tau in range(warmup):
            runtime.stage_batch(st["pool"], st["blk"], st["te"], tls[tau % cfg.n_steps], st["x"], st["h"])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for tau in range(steps):
            runtime.stage_batch(st["pool"], st["blk"], st["te"], tls[tau % cfg.n_steps], st["x"], st["h"])
        e1.record()
        torch.cuda.synchronize()
        out[n] = e0.elapsed_time(e1) / steps
        del st
        torch.cuda.empty_cache()
    ns = np.array(sorted(out), dtype=np.float64)
    ts = np.array([out[n] for n in sorted(out)])
    b, a = np.polyfit(ns, ts, 1)
    return out, float(a), float(b)


def run_placement(cfg, a, b, n_gpus=24, max_discrepancy=2):
    """Streams of one model admitted on a pool of GPUs by the joint placement
    against an equal split (each stream its own group of GPUs), for several
    chunk-interval SLOs, with the measured batch cost a + b n."""
    from autoregressive_denoising_dit_amd.sched import Scheduler, admitted_streams
    # one memory position per virtual rank: HBM left after weights over the KV
    # rings of the largest rank (ring slots of L tokens x 2D per stage, bf16)
    slot_bytes = cfg.tokens * 2 * cfg.hidden * 2
    rows = []
    stages = cfg.n_blocks * cfg.n_steps
    alone_one_gpu = cfg.n_blocks * (a + b * cfg.n_steps)      # whole stream on one GPU
    for frac in (0.7, 0.4, 0.3, 0.15, 0.08):
        slo = alone_one_gpu * frac * 1.0001
        probe = Scheduler(n_gpus, 1 << 20, cfg.n_blocks, cfg.n_steps, slo, a, b, max_discrepancy)
        R = probe.split()
        if R == 0:
            continue
        row = {"slo_ms": round(slo, 2), "ranks_per_stream": R, "equal_split_streams": n_gpus // R}
        # joint placement with the fewest ranks, and with four times finer ranks
        # (one discrepancy: the search over many small ranks grows quickly)
        for key, nr, disc in (("joint_streams", 0, max_discrepancy), ("joint_streams_fine", min(stages, 4 * R), 1)):
            per_rank = -(-stages // (nr or R)) * (cfg.window + 1) * slot_bytes
            positions = max(1, int(200e9 // per_rank))
            row[key] = admitted_streams(Scheduler(n_gpus, positions, cfg.n_blocks, cfg.n_steps, slo, a, b, disc, nr))
            row[key.replace("streams", "ranks")] = nr or R
        rows.append(row)
    return rows


def run_placed_bench(cfg, n_streams=3, ranks_per_stream=4, measured=24, sweep=(1, 2, 4, 8, 12)):
    """The stage groups the joint placement puts on this GPU, run as the stage
    pipeline (runner.PlacedRunner): the block-batch cost a + b n is fitted on
    this GPU first, the placement admits streams on one GPU under an SLO of
    1.05 x the modelled cycle of n_streams whole streams (so exactly that many
    fit), and the streams start at offset phases.  After the pipeline has
    filled, each tick's time is measured and compared with the cycle the
    placement assumed and with the SLO."""
    import torch
    from autoregressive_denoising_dit_amd import runtime
    from autoregressive_denoising_dit_amd.runner import PlacedRunner, model_cycle_ms, rank_stages
    from autoregressive_denoising_dit_amd.sched import Scheduler
    times, a, b = run_batch_sweep(cfg, sizes=sweep)
    B, S, W, D, F, H, d = cfg.n_blocks, cfg.n_steps, cfg.window, cfg.hidden, cfg.ffn, cfg.heads, cfg.head_dim
    N = B * S
    full = {sg: list(range(N)) for sg in range(n_streams)}
    slo = 1.05 * model_cycle_ms(full, S, a, b)
    sched = Scheduler(1, 64, B, S, slo, a, b, 2, ranks_per_stream)
    ranks, sg = [], 0
    while True:
        gpus = sched.admit(sg)
        if gpus is None:
            break
        ranks += [(sg, *rank_stages(N, len(gpus), r)) for r in range(len(gpus))]
        sg += 1
    admitted = sg
    _log(f"placed: a = {a:.3f} ms, b = {b:.3f} ms, SLO {slo:.1f} ms, {admitted} stream(s) admitted")
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    td = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32

    def rn(*shape, dtype=torch.float32, std=0.02):
        return (torch.randn(*shape, generator=g, device="cuda") * std).to(dtype).contiguous()

    pool = runtime.Pool(admitted, B, S, W + 1, cfg.grid, H, d, cfg.n_ctx, runtime.ps_dtype(cfg.dtype))
    blocks, keep = [], []
    for bi in range(B):
        w = {"wqkv": rn(3 * D, D, dtype=td), "wo": rn(D, D, dtype=td), "wq2": rn(D, D, dtype=td),
             "wkv2": rn(2 * D, D, dtype=td), "wo2": rn(D, D, dtype=td), "w1": rn(F, D, dtype=td),
             "w2": rn(D, F, dtype=td), "bqkv": rn(3 * D), "bo": rn(D), "bq2": rn(D), "bkv2": rn(2 * D),
             "bo2": rn(D), "b1": rn(F), "b2": rn(D), "tmod": rn(6, D)}
        blk = runtime.Block(w, D, H, d, F, bi, runtime.ps_dtype(cfg.dtype))
        for s_ in range(admitted):
            pool.context_set(blk, s_, rn(cfg.n_ctx, D, dtype=td, std=1.0))
        blocks.append(blk)
        keep.append(w)
    tw = {"wt1": rn(D, 256), "bt1": rn(D), "wt2": rn(D, D), "bt2": rn(D), "wp": rn(6 * D, D), "bp": rn(6 * D)}
    te = runtime.TimeEmbed(tw, D, capacity=16)
    starts = {s_: 2 * s_ for s_ in range(admitted)}
    fill = max(starts.values()) + N - 1          # first tick with every stage busy
    n_tick = fill + measured
    n_chunks = n_tick
    x = {s_: rn(n_chunks, cfg.tokens, D, std=1.0) for s_ in range(admitted)}
    runner = PlacedRunner(pool, blocks, te, cfg.timesteps, W, ranks, starts, n_chunks)
    torch.cuda.synchronize()
    ev = {}
    for tau in range(n_tick):
        if tau == fill:
            ev[tau] = torch.cuda.Event(enable_timing=True)
            ev[tau].record()
        runner.run_tick(tau, x)
        if tau >= fill:
            ev[tau + 1] = torch.cuda.Event(enable_timing=True)
            ev[tau + 1].record()
    torch.cuda.synchronize()
    assert all(torch.isfinite(v).all().item() for v in x.values()), "non-finite latents"
    ticks = sorted(ev[t].elapsed_time(ev[t + 1]) for t in range(fill, n_tick))
    model = runner.model_cycle_ms(a, b)
    mean = sum(ticks) / len(ticks)
    return {"batch_ms": {str(n): round(t, 3) for n, t in times.items()},
            "fit_ms": {"fixed": round(a, 4), "per_task": round(b, 4)},
            "slo_ms": round(slo, 3), "streams_admitted": admitted, "ranks_per_stream": ranks_per_stream,
            "start_ticks": starts, "tasks_per_block_batch": runner.tick_blocks[0],
            "cycle_ms": {"measured_mean": round(mean, 3), "measured_p90": round(ticks[(9 * len(ticks)) // 10], 3),
                         "model": round(model, 3), "measured_over_model": round(mean / model, 4)},
            "slo_violations": sum(1 for t in ticks if t > slo), "ticks_measured": len(ticks),
            "chunk_interval_ms_per_stream": round(mean, 3)}


def run_graph_bench(cfg, reps=50):
    """One step of the path -- at c2 a stage batch and its Euler update, at
    c3 / c4 one steady-state tick of the staggered schedule (all blocks, then
    Euler) -- run eagerly and as a HIP graph captured once and replayed, the
    same work each time, on one stream set up by an uncaptured warm-up."""
    import torch
    from autoregressive_denoising_dit_amd import runtime
    stream = torch.cuda.Stream()
    if cfg.n_blocks == 1:
        st = setup_stage(cfg, cfg.batch)
        tl = stage_tasks(cfg, cfg.batch, 0)
        dts = [cfg.timesteps[t.step] - (cfg.timesteps[t.step + 1] if t.step + 1 < cfg.n_steps else 0.0) for t in tl]

        def step():
            runtime.stage_batch(st["pool"], st["blk"], st["te"], tl, st["x"], st["h"])
            runtime.euler_update(st["xe"], st["h"], dts, cfg.tokens, cfg.hidden)
        keep = st
    else:
        from autoregressive_denoising_dit_amd.schedule import StaggeredRunner
        g_ = torch.Generator(device="cuda")
        g_.manual_seed(0)
        td = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        D, F, H, d, B, S, W, k = cfg.hidden, cfg.ffn, cfg.heads, cfg.head_dim, cfg.n_blocks, cfg.n_steps, cfg.window, cfg.k

        def rn(*shape, dtype=torch.float32, std=0.02):
            return (torch.randn(*shape, generator=g_, device="cuda") * std).to(dtype).contiguous()
        pool = runtime.Pool(1, B, S, W + k, cfg.grid, H, d, cfg.n_ctx, runtime.ps_dtype(cfg.dtype), check_slots=False)
        blocks, ws = [], []
        for b in range(B):
            w = {"wqkv": rn(3 * D, D, dtype=td), "wo": rn(D, D, dtype=td), "wq2": rn(D, D, dtype=td),
                 "wkv2": rn(2 * D, D, dtype=td), "wo2": rn(D, D, dtype=td), "w1": rn(F, D, dtype=td),
                 "w2": rn(D, F, dtype=td), "bqkv": rn(3 * D), "bo": rn(D), "bq2": rn(D), "bkv2": rn(2 * D),
                 "bo2": rn(D), "b1": rn(F), "b2": rn(D), "tmod": rn(6, D)}
            blk = runtime.Block(w, D, H, d, F, b, runtime.ps_dtype(cfg.dtype))
            pool.context_set(blk, 0, rn(cfg.n_ctx, D, dtype=td, std=1.0))
            blocks.append(blk)
            ws.append(w)
        tw = {"wt1": rn(D, 256), "bt1": rn(D), "wt2": rn(D, D), "bt2": rn(D), "wp": rn(6 * D, D), "bp": rn(6 * D)}
        te = runtime.TimeEmbed(tw, D, capacity=16)
        runner = StaggeredRunner(pool, blocks, te, cfg.timesteps, W, k, 1)
        tau = S + W + 2
        n_chunks = k * (tau + 1)
        x = rn(n_chunks, 1, cfg.tokens, D, std=1.0)

        def step():
            runner.run_tick(tau, x, n_chunks)
        keep = (pool, blocks, ws, te, runner, x)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for _ in range(3):          # warm-up: workspaces and timestep rows on this stream
            step()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            step()
        e1.record(stream)
    torch.cuda.synchronize()
    eager = e0.elapsed_time(e1) / reps
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        step()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        graph.replay()
        e0.record(stream)
        for _ in range(reps):
            graph.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    replay = e0.elapsed_time(e1) / reps
    del keep
    return {"eager_ms": round(eager, 4), "graph_ms": round(replay, 4), "graph_over_eager": round(replay / eager, 4),
            "reps": reps}


def stage_tasks(cfg, n_tasks, tau, base_chunk=100):
    """Task i: stream i at step (tau + i) mod S, a steady-state chunk with a full window."""
    from autoregressive_denoising_dit_amd import runtime
    R = cfg.window + 1
    out = []
    for i in range(n_tasks):
        s = (tau + i) % cfg.n_steps
        c = base_chunk + tau
        out.append(runtime.make_task(i, c, s, cfg.timesteps[s], c % R,
                                     [(c - cfg.window + j) % R for j in range(cfg.window)]))
    return out


def run_stage_bench(cfg, n_tasks, steps, warmup, overlap=1):
    """Stage batches plus their Euler updates, `steps` timed after `warmup`.
    With overlap = k > 1, step tau runs on stream tau mod k with its own output
    and latent buffers: consecutive batches of the schedule touch different
    (stream, step) regions of the pool, so they may overlap on the device."""
    import torch
    from autoregressive_denoising_dit_amd import _lib, runtime
    _log(f"setting up {cfg.name}: {n_tasks} tasks per batch, {overlap} stream(s)")
    st = setup_stage(cfg, n_tasks)
    L, D = cfg.tokens, cfg.hidden
    task_lists = [stage_tasks(cfg, n_tasks, tau) for tau in range(cfg.n_steps)]
    dts = [[cfg.timesteps[t.step] - (cfg.timesteps[t.step + 1] if t.step + 1 < cfg.n_steps else 0.0)
            for t in tl] for tl in task_lists]
    main = torch.cuda.current_stream()
    streams = [main] + [torch.cuda.Stream() for _ in range(overlap - 1)]
    hs = [st["h"]] + [torch.empty_like(st["h"]) for _ in range(overlap - 1)]
    xes = [st["xe"]] + [st["xe"].clone() for _ in range(overlap - 1)]

    def step(tau):
        k = tau % overlap
        tl = task_lists[tau % cfg.n_steps]
        runtime.stage_batch(st["pool"], st["blk"], st["te"], tl, st["x"], hs[k], cuda_stream=streams[k])
        runtime.euler_update(xes[k], hs[k], dts[tau % cfg.n_steps], L, D, cuda_stream=streams[k])

    def fork(ev):
        for s_ in streams[1:]:
            s_.wait_event(ev)

    def join():
        for s_ in streams[1:]:
            e = torch.cuda.Event()
            e.record(s_)
            main.wait_event(e)

    for tau in range(warmup):
        step(tau)
    join()
    # timed region: no per-kernel events (they add a gap between kernels)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(main)
    fork(ev[0])
    for tau in range(steps):
        step(tau)
        if overlap == 1:
            ev[tau + 1].record(main)
    if overlap > 1:
        join()
        ev[steps].record(main)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for h_ in hs:
        assert torch.isfinite(h_).all().item(), "non-finite stage output"
    sec = (t1 - t0) / steps
    if overlap == 1:
        per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    else:
        per_step = [ev[0].elapsed_time(ev[steps]) / steps] * steps
    # the same steps again with a HIP event pair around every kernel, recorded
    # by the library on the stream the kernel runs on: per-kernel durations
    _lib.trace_enable(True)
    for tau in range(steps):
        step(tau)
    join()
    torch.cuda.synchronize()
    trace = _lib.trace_read()
    _lib.trace_enable(False)
    return sec, trace, per_step


def shader_clock_mhz():
    """Current shader clock from the driver's DPM table (best effort; None if unreadable)."""
    import glob
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            for line in open(path):
                if line.strip().endswith("*"):
                    return int(line.split(":")[1].strip().rstrip("*").strip().lower().replace("mhz", ""))
        except (OSError, ValueError, IndexError):
            continue
    return None


def copy_calibration(nbytes=1 << 30, reps=3):
    """A plain device copy of known size: the reference that scales the HBM
    byte counters (FETCH_SIZE, WRITE_SIZE) of a profiling run to bytes."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").random_(0, 255)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


def _short_kernel(name):
    for key in ("k_attn", "k_gemm", "k_layernorm_n", "k_layernorm", "k_euler", "k_modulation", "k_put_tasks",
                "k_entry_load", "k_gemv", "copy"):
        if key in name:
            return key
    return None


def pmc_summary(dirs):
    """Per-dispatch averages of the counters of rocprofv3 --pmc CSV output, per
    kernel.  Self- and cross-attention share one kernel; in a step the
    self-attention launch comes first, so attention dispatches alternate."""
    import csv
    import glob
    per = {}
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for row in csv.DictReader(open(path)):
                k = _short_kernel(row["Kernel_Name"])
                if k is None:
                    continue
                if k == "k_gemm":
                    # the epilogue is the last template argument: k_gemm<T, E>
                    k = "k_gemm_E" + row["Kernel_Name"].split("Li", 1)[1][:1] if "Li" in row["Kernel_Name"] else k
                key = (k, int(row["Dispatch_Id"]))
                per.setdefault(key, {})
                c = row["Counter_Name"]
                per[key][c] = per[key].get(c, 0.0) + float(row["Counter_Value"])
    out = {}
    attn = sorted(d for (k, d) in per if k == "k_attn")
    for (k, did), cs in per.items():
        name = k
        if k == "k_attn":
            name = "attn_self" if attn.index(did) % 2 == 0 else "attn_cross"
        agg = out.setdefault(name, {"dispatches": 0})
        agg["dispatches"] += 1
        for c, v in cs.items():
            agg[c] = agg.get(c, 0.0) + v
    for name, agg in out.items():
        n = agg["dispatches"]
        for c in list(agg):
            if c != "dispatches":
                agg[c] = round(agg[c] / n, 3)
        # Matrix-core utilisation: SQ_VALU_MFMA_BUSY_CYCLES sums busy cycles over
        # all SIMDs; GRBM_GUI_ACTIVE sums the GPU's active cycles over the XCDs.
        if "SQ_VALU_MFMA_BUSY_CYCLES" in agg and agg.get("GRBM_GUI_ACTIVE"):
            cyc = agg["GRBM_GUI_ACTIVE"] / MI355X_XCDS
            agg["mfma_busy_frac"] = round(agg["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * MI355X_SIMDS), 4)
            agg["active_cycles_per_xcd"] = round(cyc)
    print(json.dumps(out, indent=1, sort_keys=True), flush=True)


def trace_summary(dirs):
    """Per-kernel dispatch counts and durations from rocprofv3 --kernel-trace
    CSV output (the kernel_trace.csv of each directory).  Self- and
    cross-attention share one kernel; within a stage call the self-attention
    launch comes first, so attention dispatches alternate."""
    import csv
    import glob
    rows = []
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
            for r in csv.DictReader(open(path)):
                rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]))
    rows.sort()
    out = {}
    attn_seen = 0
    for (t0, t1, name) in rows:
        k = _short_kernel(name) or name[:60]
        if k == "k_gemm" and "Li" in name:
            k = "k_gemm_E" + name.split("Li", 1)[1][:1]
        if k == "k_attn":
            k = "attn_self" if attn_seen % 2 == 0 else "attn_cross"
            attn_seen += 1
        agg = out.setdefault(k, {"dispatches": 0, "total_ms": 0.0})
        agg["dispatches"] += 1
        agg["total_ms"] += (t1 - t0) * 1e-6
    for agg in out.values():
        agg["avg_ms"] = round(agg["total_ms"] / agg["dispatches"], 4)
        agg["total_ms"] = round(agg["total_ms"], 3)
    print(json.dumps(out, indent=1, sort_keys=True), flush=True)


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None when there is none or the kernel's source changed since it was taken.
    profiles/traffic.json: {"workload", "copy_fetch_scale", "copy_write_scale",
    "kernels": {name: {"fetch_kib", "write_kib", "sources": {path: sha256}}}}."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    doc = json.load(open(path))
    rec = doc.get("kernels", {}).get(kernel)
    if rec is None:
        return None
    for rel, digest in rec["sources"].items():
        f = os.path.join(root, rel)
        if not os.path.exists(f) or hashlib.sha256(open(f, "rb").read()).hexdigest() != digest:
            return None
    kib = rec["fetch_kib"] * doc["copy_fetch_scale"] + rec["write_kib"] * doc["copy_write_scale"]
    return int(round(kib * 1024))


def cpu_baseline(cfg, n_read, budget_s=30.0):
    """The float64 CPU oracle on whole stage tasks of the workload (a bounded
    sample of about ten seconds): oracle stage tasks per second."""
    import numpy as np
    import oracle
    from synthetic import inputs, stage_flops
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    _log("cpu baseline: generating one block's weights")
    w = inputs.block_weights(cfg, 0, 0)
    tw = inputs.time_weights(cfg, 0)
    L, H, d = cfg.tokens, cfg.heads, cfg.head_dim
    h = inputs.hidden_rows(cfg, 1, 0)
    prior = [inputs.cache_entry(cfg, 0, 0, 0, j, 0) for j in range(n_read)]
    ctx_kv = oracle.context_kv(inputs.context(cfg, 0, 0), w, H)
    e = oracle.time_embedding(cfg.timesteps[0], tw)
    # sample: whole stage tasks (every query row, the full window), repeated
    # until about ten seconds of CPU work have been timed
    done, dt = 0, 0.0
    while done == 0 or (dt < 10.0 and dt * (done + 1) / done < budget_s):
        _log(f"cpu baseline: oracle stage task {done + 1}")
        t0 = time.perf_counter()
        oracle.block_task(h, e, w, 10, prior, ctx_kv, cfg.grid, H)
        dt += time.perf_counter() - t0
        done += 1
    return {"value": done / dt, "unit": "tasks/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} whole {cfg.name} stage task(s) (all {L} query rows, {n_read} prior chunks "
                      f"+ own chunk of keys, {cfg.n_ctx} context tokens) in float64 NumPy: "
                      f"{dt:.1f} s measured"}


def cpu_baseline_interval(cfg):
    """The oracle's chunk interval of the staggered schedule, extrapolated from
    timed whole stage tasks: a chunk takes one task per (block, step), and the
    oracle runs them one after another."""
    r = cpu_baseline(cfg, cfg.window)
    per_chunk = cfg.n_blocks * cfg.n_steps
    return {"value": round(per_chunk / r["value"] * 1e3, 1), "unit": "ms per chunk", "cores": r["cores"],
            "kind": "oracle",
            "sample": r["sample"] + f"; extrapolated to the {per_chunk} tasks (blocks x steps) of one chunk"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c5", choices=["c2", "c5", "c3", "c4", "placement", "placed"],
                    help="c5 (default) / c2: one stage batch per step; c3 / c4: the staggered schedule "
                         "over all blocks and steps, reporting the chunk interval; placement: block-batch "
                         "cost sweep at the 1.3B and 5B shapes and the joint placement it drives; placed: "
                         "the stage groups placed on this GPU run as the stage pipeline at the 1.3B shape, "
                         "measured cycle against the placement's model")
    ap.add_argument("--overlap", type=int, default=1,
                    help="c5 / c2: streams that consecutive stage batches alternate over (1 = one stream)")
    ap.add_argument("--graph", action="store_true",
                    help="c2 / c3 / c4: time one step (c2) or one tick (c3, c4) eagerly and as a replayed HIP graph")
    ap.add_argument("--no-timeshared", action="store_true",
                    help="c5: leave out the c3 / c4 chunk intervals that the default line also carries")
    ap.add_argument("--groups", type=int, default=2,
                    help="c3 / c4: run each tick's tasks as this many groups of steps on concurrent streams")
    ap.add_argument("--head", action="store_true",
                    help="c3 / c4: run on latent patches with the patch embedding and output head")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (reference for the HBM byte counters)")
    ap.add_argument("--pmc-summary", nargs="+", metavar="DIR",
                    help="only summarise rocprofv3 --pmc CSV output per kernel and exit")
    ap.add_argument("--trace-summary", nargs="+", metavar="DIR",
                    help="only summarise rocprofv3 --kernel-trace CSV output per kernel and exit")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the stage path runs on one GPU only (no multi-GPU path); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from synthetic import get, stage_flops
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.workload == "placement":
        res = {}
        for name in ("c3", "c4"):
            cfg = get(name)
            times, a, b = run_batch_sweep(cfg)
            res[cfg.name] = {"batch_ms": {str(n): round(t, 3) for n, t in times.items()},
                             "fit_ms": {"fixed": round(a, 4), "per_task": round(b, 4)},
                             "placement_24_gpus": run_placement(cfg, a, b)}
        print(json.dumps({"metric": "streams admitted on 24 GPUs, joint placement vs equal split",
                          "n_gpus": 1, "data": "synthetic; batch costs measured on this GPU", **res}), flush=True)
        return
    if args.graph:
        cfg = get(args.workload)
        res = run_graph_bench(cfg)
        print(json.dumps({"metric": "one step as a HIP graph vs eager launches", "n_gpus": 1, "dtype": cfg.dtype,
                          "config": {"workload": cfg.name, "unit": "stage step" if cfg.n_blocks == 1 else "tick"},
                          **res}), flush=True)
        return
    if args.workload == "placed":
        cfg = get("c3")
        res = run_placed_bench(cfg)
        print(json.dumps({"metric": "measured vs modelled cycle of the stage groups placed on one GPU",
                          "n_gpus": 1, "dtype": cfg.dtype,
                          "data": "synthetic (seeded random-init weights, N(0,1) latents and contexts)",
                          "config": {"workload": "placed_wan13b_pipeline", "blocks": cfg.n_blocks,
                                     "steps": cfg.n_steps, "window": cfg.window, "tokens_per_chunk": cfg.tokens,
                                     "hidden": cfg.hidden},
                          **res}), flush=True)
        return
    if args.workload in ("c3", "c4"):
        cfg = get(args.workload)
        interval, tick, done, per_tick = run_stagger_bench(cfg, with_head=args.head, groups=args.groups)
        per_chunk = cfg.n_blocks * cfg.n_steps * stage_flops(cfg, cfg.window)
        print(json.dumps({
            "metric": "steady-state chunk interval (ms), staggered schedule, one stream",
            "value": round(interval, 3), "unit": "ms", "n_gpus": 1, "higher_is_better": False,
            "dtype": cfg.dtype, "data": "synthetic (seeded random-init weights, N(0,1) latents and contexts)",
            "config": {"workload": cfg.name, "blocks": cfg.n_blocks, "steps": cfg.n_steps, "k": cfg.k,
                       "window": cfg.window, "tokens_per_chunk": cfg.tokens, "hidden": cfg.hidden,
                       "head": bool(args.head), "latent_dim": cfg.latent_dim if args.head else None,
                       "groups": args.groups},
            "chunks_measured": done, "tick_ms": round(tick, 3),
            "stage_tasks_per_s": round(cfg.n_blocks * cfg.n_steps * cfg.k / (tick * 1e-3), 1),
            "mfma_frac": round(per_chunk / (interval * 1e-3) / PEAK[cfg.dtype], 4),
            "kernel_ms_per_tick": per_tick,
            **({} if args.no_cpu_baseline else {"cpu_baseline": cpu_baseline_interval(cfg)}),
        }), flush=True)
        return
    cfg = get(args.workload)
    n_tasks = cfg.batch
    n_read = cfg.window
    sec, trace, per_step = run_stage_bench(cfg, n_tasks, args.steps, args.warmup, args.overlap)
    sclk = shader_clock_mhz()
    flops_step = n_tasks * stage_flops(cfg, n_read)
    peak = PEAK[cfg.dtype]
    work = kernel_work(cfg, n_tasks, n_read)
    kv = cache_bytes(cfg, n_tasks, n_read)
    kernels = {}
    for name, (launches, ms) in trace.items():
        avg_ms = ms / max(launches, 1)
        rec = {"launches": launches, "avg_ms": round(avg_ms, 4)}
        if name in work:
            kind, amount = work[name]
            if kind == "flop":
                rec["tflops"] = round(amount / (avg_ms * 1e-3) / 1e12, 1)
            else:
                rec["gbs"] = round(amount / (avg_ms * 1e-3) / 1e9, 1)
        if name in kv:
            rec["kv_gbs"] = round(kv[name] / (avg_ms * 1e-3) / 1e9, 1)
        kernels[name] = rec
    dom = max((n for n in trace if n in work), key=lambda n: trace[n][1])
    kind, amount = work[dom]
    avg_s = trace[dom][1] / trace[dom][0] * 1e-3
    if kind == "flop":
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(amount / avg_s / 1e12, 2), "peak": peak / 1e12,
                "unit": "TFLOP/s", "frac": round(amount / avg_s / peak, 4)}
    else:
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(amount / avg_s / 1e9, 1), "peak": HBM_PEAK / 1e9,
                "unit": "GB/s", "frac": round(amount / avg_s / HBM_PEAK, 4)}
    # measured HBM bytes per launch of the dominant kernel (profiles/traffic.json)
    roof["traffic"] = measured_traffic(dom)
    out = {
        "metric": "stage tasks/sec + steady-state chunk interval (ms) on 1 MI355X; % MFMA peak",
        "value": round(n_tasks / sec, 2),
        "unit": "tasks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded random-init weights, N(0,1) latents, contexts and pre-filled noisy KV)",
        "config": {"workload": cfg.name, "tasks_per_batch": n_tasks, "tokens_per_chunk": cfg.tokens,
                   "hidden": cfg.hidden, "heads": cfg.heads, "head_dim": cfg.head_dim, "ffn": cfg.ffn,
                   "window": cfg.window, "ctx_tokens": cfg.n_ctx, "steps_mixed": cfg.n_steps,
                   "overlap_streams": args.overlap},
        # each stream's chunk needs one task per denoising step at this block
        "chunk_interval_ms": round(sec * 1e3 * cfg.n_steps, 3),
        "mfma_frac": round(flops_step / sec / peak, 4),
        "stage_tflops": round(flops_step / sec / 1e12, 1),
        # HIP events between consecutive steps of the timed region
        "step_ms": {"median": round(per_step[len(per_step) // 2], 3), "p10": round(per_step[len(per_step) // 10], 3),
                    "p90": round(per_step[min(len(per_step) - 1, (9 * len(per_step)) // 10)], 3)},
        "sclk_mhz_after": sclk,
        "kernels": kernels,
        "roofline": roof,
    }
    if args.workload == "c5" and not args.no_timeshared:
        # the time-shared configurations, measured after the timed steps: the
        # staggered schedule over all blocks and steps of one stream
        for name in ("c3", "c4"):
            tcfg = get(name)
            _log(f"time-shared {name}: staggered schedule, {args.groups} group(s)")
            interval, tick, done, _ = run_stagger_bench(tcfg, measured=32, groups=args.groups)
            per_chunk = tcfg.n_blocks * tcfg.n_steps * stage_flops(tcfg, tcfg.window)
            out[f"{name}_chunk_interval_ms"] = round(interval, 3)
            out[f"{name}_mfma_frac"] = round(per_chunk / (interval * 1e-3) / PEAK[tcfg.dtype], 4)
        out["timeshared_groups"] = args.groups
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, n_read)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
