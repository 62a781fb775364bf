"""Parity of the HIP path (through the C ABI) with the float64 CPU oracle.

Bar: max |err| / RMS(ref) <= 3e-2 with bf16 operands and <= 1e-4 with fp32
operands, on every tensor compared (stage output, its branch delta and the
cache entries written; with the probe entry point also each kernel's own
output)."""
import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
from autoregressive_denoising_dit_amd import _lib, runtime
from autoregressive_denoising_dit_amd._lib import PsError, PS_ERR_SLOT_CONFLICT, PS_ERR_INVALID_ARG
from synthetic import C1, C2, C3, C4, C5, inputs, with_
from tests.gpu_util import (StageCase, host, make_block, make_pool, make_te, rel_err, say, to_dev, tol)

pytestmark = pytest.mark.gpu


def _check_case(case, task_ids=None, rows=None, delta=True):
    """The stage output h_out and the cache entries written, at the bound
    (the bound is stated for outputs); with ``delta`` also the branch delta h_out - h_in,
    which is small next to the residual stream."""
    cfg, L = case.cfg, case.cfg.tokens
    t = tol(cfg)
    ids = list(range(len(case.tasks))) if task_ids is None else task_ids
    for i in ids:
        got = case.gpu_h_out[i * L:(i + 1) * L]
        h = case.h_in[i * L:(i + 1) * L]
        if rows is not None:
            got, h = got[rows], h[rows]
        ref = case.ref_h_out[i]
        e_out = rel_err(got, ref)
        e_delta = rel_err(got - h, ref - h)
        say(f"task {i} {case.tasks[i]}: h_out err {e_out:.2e}, branch delta err {e_delta:.2e}")
        assert e_out <= t, (i, e_out)
        assert e_delta <= t or not delta, (i, e_delta)
        key = (case.tasks[i][0], case.tasks[i][1], case.tasks[i][2])
        if key in case.ref_kv:
            k_ref, v_ref = case.ref_kv[key]
            k_got, v_got = case.gpu_kv[key]
            ek, ev = rel_err(k_got, k_ref), rel_err(v_got, v_ref)
            say(f"task {i}: cache k err {ek:.2e}, v err {ev:.2e}")
            assert ek <= t and ev <= t


UNIT_ROUNDOFF = {"bf16": 2.0 ** -8, "fp32": 2.0 ** -24}   # round to nearest, 8 / 24 significant bits


def _probe_err(got, ref, allow):
    """max(|got - ref| - allow, 0) / RMS(ref), elementwise allowance."""
    assert got.shape == ref.shape and np.all(np.isfinite(got))
    return float(np.maximum(np.abs(got - ref) - allow, 0.0).max() / np.sqrt(np.mean(ref ** 2)))


def _check_probe(case, task_ids=None, rows=None):
    """Each kernel's output in the chain of one stage call
    (ps_stage_batch_probe) against the oracle's matching intermediate, task by
    task, at the plain bound.  A stored member carries its own rounding, at
    most the unit roundoff of its storage type times the value (2^-8 in bf16,
    2^-24 in fp32); that is taken off each element's error before the bound
    max|err| / RMS(ref) <= tol applies.  The same holds for the branch deltas
    h1 - h and h2 - h1, whose operands are stored fp32 values that are large
    next to the delta.  The queries are stored times log2(e)/sqrt(d), which is
    divided out.  In the chain every kernel also inherits the rounding of its
    inputs; each kernel on its own, on identical inputs, is scored in
    test_gpu_kernels.py."""
    cfg, L = case.cfg, case.cfg.tokens
    t = tol(cfg)
    u32 = UNIT_ROUNDOFF["fp32"]
    qscale = math.log2(math.e) / math.sqrt(cfg.head_dim)
    ids = list(range(len(case.tasks))) if task_ids is None else task_ids
    for i in ids:
        tr = case.ref_trace[i]
        sel = torch.arange(i * L, (i + 1) * L, device="cuda") if rows is None else \
            torch.as_tensor(i * L + np.asarray(rows), device="cuda")
        got_h = {}
        for name in _lib.PROBE_FIELDS:
            got = host(case.gpu_probe[name].index_select(0, sel))
            ref = tr[name] if rows is None or name not in ("y1", "q") else tr[name][rows]
            if name in ("q", "q2"):
                got = got / qscale
            u = u32 if name in _lib.PROBE_FP32 else UNIT_ROUNDOFF[cfg.dtype]
            err = _probe_err(got, ref, u * np.abs(ref))
            say(f"task {i} probe {name}: err {err:.2e} (plain {rel_err(got, ref):.2e})")
            assert err <= t, (i, name, err)
            got_h[name] = got
        # the gated / plain branch deltas, which are small next to the residual stream
        h = case.h_in[i * L:(i + 1) * L] if rows is None else case.h_in[i * L:(i + 1) * L][rows]
        for name, a, b, ra, rb, allow in (
                ("h1 - h", got_h["h1"], h, tr["h1"], h, u32 * np.abs(tr["h1"])),
                ("h2 - h1", got_h["h2"], got_h["h1"], tr["h2"], tr["h1"], u32 * (np.abs(tr["h2"]) + np.abs(tr["h1"])))):
            e = _probe_err(a - b, ra - rb, allow)
            say(f"task {i} probe {name}: err {e:.2e} (plain {rel_err(a - b, ra - rb):.2e})")
            assert e <= t, (i, name, e)


# ----------------------------------------------------------------- pieces
@pytest.mark.parametrize("cfg", [C1, C2], ids=["fp32_d128", "w1536"])
def test_time_embedding(cfg):
    tw = inputs.time_weights(cfg, 0)
    te = make_te(cfg, tw, capacity=2)
    for t in (1.0, 0.75, 0.3, 1.0, 0.0):   # more distinct t than capacity: eviction path
        say("time embed", cfg.name, t)
        got = host(te.get(t))
        ref = oracle.time_embedding(t, tw)
        assert rel_err(got, ref) <= 1e-4


@pytest.mark.parametrize("cfg", [C1, C2], ids=["fp32", "bf16"])
def test_context_keys_values(cfg):
    w = inputs.block_weights(cfg, 0, 0)
    pool = make_pool(cfg, n_streams=2, n_blocks=1)
    blk = make_block(cfg, w)
    td = runtime.TORCH_DTYPE[runtime.ps_dtype(cfg.dtype)]
    for sg in (1, 0):
        ctx = inputs.context(cfg, sg, 0)
        say("context", cfg.name, sg)
        pool.context_set(blk, sg, to_dev(ctx, td))
        k, v = pool.context_fetch(sg, 0, cfg.n_ctx)
        rk, rv = oracle.context_kv(ctx, w, cfg.heads)
        # one GEMM, then the rounding of its output to the compute dtype (at
        # most 2^-8 / 2^-24 of each value, taken off as in the probe checks);
        # what remains is fp32 accumulation error, far inside the bound, so a
        # third of it is required
        u = UNIT_ROUNDOFF[cfg.dtype]
        ek = _probe_err(host(k), rk, u * np.abs(rk))
        ev = _probe_err(host(v), rv, u * np.abs(rv))
        say(f"context k err {ek:.2e}, v err {ev:.2e} (plain {rel_err(host(k), rk):.2e}, {rel_err(host(v), rv):.2e})")
        assert ek <= tol(cfg) / 3 and ev <= tol(cfg) / 3


@pytest.mark.parametrize("vdt", [torch.float32, torch.bfloat16])
def test_euler_update(vdt):
    L, D, n = 64, 128, 3
    r = np.random.default_rng(3)
    x = r.standard_normal((n * L, D)).astype(np.float32)
    v = r.standard_normal((n * L, D)).astype(np.float32)
    dt = [0.5, 0.25, 0.125]
    xd, vd = to_dev(x, torch.float32), to_dev(v, vdt)
    say("euler", vdt)
    runtime.euler_update(xd, vd, dt, L, D)
    vv = host(vd)
    ref = x.astype(np.float64) - np.repeat(np.array(dt), L)[:, None] * vv
    assert rel_err(host(xd), ref) <= 1e-6


def test_pool_load_fetch_roundtrip():
    cfg = C1
    pool = make_pool(cfg, n_streams=1, n_blocks=1)
    k, v = inputs.cache_entry(cfg, 0, 0, 1, 5, 0)
    say("pool roundtrip")
    pool.load(0, 0, 1, 2, 5, to_dev(k, torch.float32), to_dev(v, torch.float32))
    k2, v2 = pool.fetch(0, 0, 1, 2)
    assert np.array_equal(host(k2), k) and np.array_equal(host(v2), v)


# ------------------------------------------------------------ stage batches
def test_stage_fp32_tiny_mixed_batch():
    """C1 shapes, fp32: tasks of different chunks, steps and window fill."""
    cfg = C1
    tasks = [(0, 0, 0, 0), (0, 3, 1, 2), (0, 2, 0, 2), (0, 1, 1, 1)]
    case = StageCase(cfg, tasks, n_slots=8).run_gpu()
    case.run_oracle()
    _check_case(case)


def test_stage_fp32_reads_same_batch_write():
    """Two chunks of one step in one batch (k = 2): chunk c + 1 reads what chunk c
    writes in the same call."""
    cfg = C1
    tasks = [(0, 4, 1, 2), (0, 5, 1, 2), (0, 2, 0, 2), (0, 3, 0, 2)]
    case = StageCase(cfg, tasks, n_slots=cfg.window + 2).run_gpu(h_out_same=True)
    case.run_oracle()
    _check_case(case)


def test_stage_bf16_tiny_shapes():
    cfg = with_(C1, dtype="bf16")
    tasks = [(0, 3, 1, 2), (1, 2, 0, 2), (0, 0, 1, 0)]
    case = StageCase(cfg, tasks, n_slots=8).run_gpu()
    case.run_oracle()
    _check_case(case)


def test_stage_fp32_widest_window():
    """The widest window the boundary allows (8 prior chunks = 9 key segments),
    next to a task with none; context of 8 tokens (one 16-byte chunk per key
    row in fp32), the smallest the pool accepts."""
    cfg = with_(C1, n_ctx=8)
    tasks = [(0, 9, 0, 8), (0, 8, 1, 8), (0, 0, 1, 0)]
    case = StageCase(cfg, tasks, n_slots=10).run_gpu()
    case.run_oracle()
    _check_case(case)


def test_stage_fp32_largest_batch():
    """32 tasks (the most one batch takes): 4 streams x 2 steps x 4 chunks, each
    chunk reading the two before it, one of them written by the same batch.
    With 64-token chunks a 256-row GEMM tile spans several tasks."""
    cfg = C1
    tasks = [(sg, c, s, 2) for sg in range(4) for s in range(2) for c in range(10, 14)]
    case = StageCase(cfg, tasks, n_slots=8).run_gpu()
    case.run_oracle(task_ids=[0, 5, 13, 22, 31])
    _check_case(case, task_ids=[0, 5, 13, 22, 31])


def test_stage_bf16_head_dim_64_ragged_context():
    """bf16 with 64-dim heads at full chunk length (ragged last key tile) and a
    context of 200 tokens (ragged last cross tile); all rows of both tasks."""
    cfg = with_(C2, hidden=512, heads=8, head_dim=64, ffn=1024, n_ctx=200)
    case = StageCase(cfg, [(0, 5, 1, 3), (1, 4, 2, 2)]).run_gpu()
    case.run_oracle()
    _check_case(case)


def test_stage_probe_kernels_bf16_small():
    """Each kernel's output on its own: a bf16 batch of two tasks of two
    streams (64-dim heads, full 1560-token chunks, a 200-token context), every
    row; the probe's h_out equals ps_stage_batch's bit for bit."""
    cfg = with_(C2, hidden=512, heads=8, head_dim=64, ffn=1024, n_ctx=200)
    tasks = [(0, 5, 1, 3), (1, 4, 2, 2)]
    plain = StageCase(cfg, tasks).run_gpu()
    case = StageCase(cfg, tasks).run_gpu(probe=True)
    assert np.array_equal(plain.gpu_h_out, case.gpu_h_out)
    case.run_oracle()
    _check_case(case)
    _check_probe(case)


def test_stage_probe_kernels_fp32_tiny():
    cfg = C1
    tasks = [(0, 0, 0, 0), (0, 3, 1, 2), (0, 2, 0, 2), (0, 1, 1, 1)]
    case = StageCase(cfg, tasks, n_slots=8).run_gpu(probe=True)
    case.run_oracle()
    _check_case(case)
    _check_probe(case)


def test_stage_probe_kernels_c2_full():
    """Each kernel's output at the 1.3B shape, batch 1, full window, every row."""
    case = StageCase(C2, [(0, 7, 2, 3)]).run_gpu(probe=True)
    case.run_oracle()
    _check_probe(case)


def test_stage_c2_single_task_full():
    """Wan2.1-1.3B-shaped stage at batch 1, full window, every output row."""
    cfg = C2
    case = StageCase(cfg, [(0, 7, 2, 3)]).run_gpu()
    case.run_oracle()
    _check_case(case)


def test_stage_batch_invariance_bitwise_c2_shape():
    """A task's stage output and cache entries do not depend on its batch: at
    the 1.3B shape, batch 1 (M = 1560 rows) and batch 2 (M = 3120) take other
    GEMM row tiles and grids, and the task's results are bitwise equal."""
    a = StageCase(C2, [(0, 7, 2, 3)]).run_gpu()
    b = StageCase(C2, [(0, 7, 2, 3), (1, 7, 1, 3)]).run_gpu()
    L = C2.tokens
    assert a.h_in.shape[0] == L and np.array_equal(a.h_in, b.h_in[:L])
    assert np.array_equal(a.gpu_h_out, b.gpu_h_out[:L])
    for x, y in zip(a.gpu_kv[(0, 7, 2)], b.gpu_kv[(0, 7, 2)]):
        assert np.array_equal(x, y)


def test_stage_c3_mixed_steps_full():
    """1.3B shape, a time-shared batch of 8 tasks: 2 chunks per step at all 4
    steps (k = 2, ring W + 2); every row of all 8 tasks."""
    cfg = C3
    tasks = []
    for s in range(4):
        for j in range(2):
            c = 2 * (5 - s) + j
            tasks.append((0, c, s, min(cfg.window, c)))
    case = StageCase(cfg, tasks, n_slots=cfg.window + 2).run_gpu()
    case.run_oracle()
    _check_case(case)


def test_stage_bf16_largest_batch_c3_shape():
    """The most tasks one batch takes (32) at the 1.3B shape: 4 streams x 4
    steps x 2 chunks, the second chunk of each pair reading the first one's
    same-batch write (M = 49920 rows: 256-row eight-wave GEMM tiles, 12480
    attention workgroups); sampled rows of three tasks, one per stream end."""
    cfg = C3
    tasks = [(sg, 2 * (5 - s) + j, s, C3.window) for sg in range(4) for s in range(4) for j in range(2)]
    assert len(tasks) == 32
    case = StageCase(cfg, tasks, n_slots=cfg.window + 2).run_gpu()
    rows = np.array([0, 255, 256, 1535, 1559])
    ids = [0, 13, 31]
    case.run_oracle(task_ids=ids, rows=rows)
    _check_case(case, task_ids=ids, rows=rows)


def test_stage_c4_full():
    """5B shape (1760-token chunks), two tasks at different steps; every row."""
    cfg = C4
    tasks = [(0, 9, 3, 3), (0, 12, 0, 3)]
    case = StageCase(cfg, tasks).run_gpu()
    case.run_oracle()
    _check_case(case)


def test_stage_c5_sixteen_streams_full_rows():
    """14B-shaped stage, the batch of 16 tasks from 16 streams at mixed steps
    that the benchmark times; every row of one task per denoising step.

    The stage output and the cache entries are held to the bound.  The branch
    delta h_out - h_in is not: at this width the bf16 storage of the block's
    intermediates alone -- the oracle's float64 chain with only those values
    rounded -- moves the delta of task 0 by 3.4e-2 of its RMS
    (test_oracle_block.py::test_bf16_storage_alone_moves_the_14b_branch_delta),
    so no bf16 implementation meets 3e-2 there.  The branches are held to the
    bound kernel by kernel on identical inputs (test_gpu_kernels.py)."""
    cfg = C5
    tasks = [(i, 10 + i // 4, (i * 3) % 4, 3) for i in range(16)]
    assert sorted(tasks[i][2] for i in range(4)) == [0, 1, 2, 3]
    case = StageCase(cfg, tasks, share_prefill=True).run_gpu()
    case.run_oracle(task_ids=[0, 1, 2, 3])
    _check_case(case, task_ids=[0, 1, 2, 3], delta=False)


def test_stage_two_frame_chunks():
    """Chunks of two latent frames (grid 2 x 24 x 32): the frame index of a
    token and the per-frame rows of the RoPE frame table; every row, with the
    probe of each kernel."""
    cfg = with_(C2, hidden=512, heads=4, head_dim=128, ffn=1024, grid=(2, 24, 32), n_ctx=64)
    case = StageCase(cfg, [(0, 5, 1, 3), (0, 6, 1, 3), (1, 2, 3, 2)], n_slots=5).run_gpu(probe=True)
    case.run_oracle()
    _check_case(case)
    _check_probe(case)


def test_stage_batch_rows_matches_stage_batch_bitwise():
    """ps_stage_batch_rows, each task's rows in a tensor of its own (task 0
    updated in place), gives ps_stage_batch's stage outputs and cache entries
    bit for bit: the rows are gathered into the workspace, run as one batch
    and scattered back.  Task 2 reads the entry task 0 writes in the batch."""
    cfg = with_(C2, hidden=512, heads=8, head_dim=64, ffn=1024, n_ctx=200)
    tasks = [(0, 5, 1, 3), (1, 4, 2, 2), (0, 6, 1, 3)]
    a = StageCase(cfg, tasks, n_slots=cfg.window + 2).run_gpu()
    b = StageCase(cfg, tasks, n_slots=cfg.window + 2)
    ps_tasks = b.setup_gpu()
    L = cfg.tokens
    rows_in = [to_dev(b.h_in[i * L:(i + 1) * L], torch.float32) for i in range(len(tasks))]
    rows_out = [rows_in[0]] + [torch.empty_like(r) for r in rows_in[1:]]
    say("stage_batch_rows", cfg.name, tasks)
    runtime.stage_batch_rows(b.pool, b.block, b.te, ps_tasks, rows_in, rows_out)
    torch.cuda.synchronize()
    for i, (sg, c, s, _) in enumerate(tasks):
        assert np.array_equal(host(rows_out[i]), a.gpu_h_out[i * L:(i + 1) * L]), i
        k, v = b.pool.fetch(sg, 0, s, c % b.R)
        assert np.array_equal(host(k), a.gpu_kv[(sg, c, s)][0]) and np.array_equal(host(v), a.gpu_kv[(sg, c, s)][1])


def test_stage_rope_tables_beyond_lds():
    """A 60 x 88 token grid: the row and column RoPE tables (3152 pairs with the
    frame rows) exceed the QKV epilogue's LDS budget, so the epilogue reads
    them from memory; every row."""
    cfg = with_(C2, hidden=512, heads=4, head_dim=128, ffn=1024, grid=(1, 60, 88), n_ctx=64)
    case = StageCase(cfg, [(0, 4, 2, 3), (1, 1, 0, 1)]).run_gpu(probe=True)
    case.run_oracle()
    _check_case(case)
    _check_probe(case)


# ------------------------------------------------------------- schedules
def _schedule_inputs(cfg, n_chunks, n_streams, seed=0):
    blocks = [inputs.block_weights(cfg, b, seed) for b in range(cfg.n_blocks)]
    tw = inputs.time_weights(cfg, seed)
    ctxs = [inputs.context(cfg, sg, seed) for sg in range(n_streams)]
    lat = {(sg, c): inputs.latent(cfg, sg, c, seed) for sg in range(n_streams) for c in range(n_chunks)}
    return blocks, tw, ctxs, lat


def _gpu_schedule(cfg, blocks, tw, ctxs, lat, n_chunks, n_streams, k, keep_pool=False, groups=1):
    from autoregressive_denoising_dit_amd.schedule import StaggeredRunner
    td = runtime.TORCH_DTYPE[runtime.ps_dtype(cfg.dtype)]
    pool = make_pool(cfg, n_streams=n_streams, n_blocks=cfg.n_blocks, n_slots=cfg.window + k)
    blks = [make_block(cfg, w, b) for b, w in enumerate(blocks)]
    te = make_te(cfg, tw)
    for b, blk in enumerate(blks):
        for sg in range(n_streams):
            pool.context_set(blk, sg, to_dev(ctxs[sg], td))
    x = torch.stack([torch.stack([to_dev(lat[(sg, c)], torch.float32) for sg in range(n_streams)])
                     for c in range(n_chunks)]).contiguous()
    run = StaggeredRunner(pool, blks, te, cfg.timesteps, cfg.window, k, n_streams, groups=groups)
    run.run(x, n_chunks)
    torch.cuda.synchronize()
    return (host(x), pool) if keep_pool else host(x)


@pytest.mark.parametrize("k,n_streams", [(1, 1), (2, 1), (1, 2)])
def test_schedule_c1_matches_oracle(k, n_streams):
    """The tiny configuration end to end (2 blocks x 2 steps, 4 chunks of 64
    tokens, window 2, fp32): staggered on the GPU vs sequential in the oracle."""
    cfg, n_chunks = C1, 4
    blocks, tw, ctxs, lat = _schedule_inputs(cfg, n_chunks, n_streams)
    say("schedule c1", k, n_streams)
    gx = _gpu_schedule(cfg, blocks, tw, ctxs, lat, n_chunks, n_streams, k)
    ox, _ = oracle.run_schedule(cfg, blocks, tw, lambda sg, c: lat[(sg, c)], ctxs, n_chunks,
                                order="sequential")
    for c in range(n_chunks):
        for sg in range(n_streams):
            e = rel_err(gx[c, sg], ox[(sg, c)])
            say(f"chunk {c} stream {sg}: x^S err {e:.2e}")
            assert e <= 1e-4


def test_schedule_batch_invariance_bitwise_c3_shape():
    """A task's result does not depend on its batch companions: the staggered
    run (batches of 8 mixed-step tasks) and k = 1 run at 1.3B width give
    bitwise equal latents (2 blocks, 5 chunks)."""
    cfg = with_(C3, n_blocks=2)
    n_chunks = 5
    blocks, tw, ctxs, lat = _schedule_inputs(cfg, n_chunks, 1)
    say("batch invariance c3 shape")
    a = _gpu_schedule(cfg, blocks, tw, ctxs, lat, n_chunks, 1, 2)
    b = _gpu_schedule(cfg, blocks, tw, ctxs, lat, n_chunks, 1, 1)
    assert np.array_equal(a, b)
    assert np.all(np.isfinite(a))


def test_schedule_bf16_c3_shape_matches_oracle():
    """The 1.3B shape in bf16 end to end at reduced depth: 2 blocks x 4 steps,
    7 chunks, k = 2 (block batches of up to 8 tasks at mixed steps, chunk c + 1
    reading chunk c's same-batch write), staggered on the GPU against the
    oracle's sequential run.  Scored at the bf16 bound: every chunk's x^S and
    x^0 - x^S, and the noisy-KV entries the run leaves in the pool (the last
    W + k chunks of every (block, step)), which carry the hand-off of noisy KV
    between chunks across blocks and steps."""
    cfg = with_(C3, n_blocks=2)
    n_chunks, k = 7, 2
    blocks, tw, ctxs, lat = _schedule_inputs(cfg, n_chunks, 1)
    say("schedule bf16 1.3B shape, 2 blocks x 4 steps, 7 chunks, k = 2")
    gx, pool = _gpu_schedule(cfg, blocks, tw, ctxs, lat, n_chunks, 1, k, keep_pool=True)
    ox, opool = oracle.run_schedule(cfg, blocks, tw, lambda sg, c: lat[(sg, c)], ctxs, n_chunks,
                                    order="sequential", k=k)
    t = tol(cfg)
    for c in range(n_chunks):
        x0 = lat[(0, c)].astype(np.float64)
        e, ed = rel_err(gx[c, 0], ox[(0, c)]), rel_err(x0 - gx[c, 0], x0 - ox[(0, c)])
        say(f"chunk {c}: x^S err {e:.2e}, x^0 - x^S err {ed:.2e}")
        assert e <= t and ed <= t
    R = cfg.window + k
    for b in range(cfg.n_blocks):
        for s in range(cfg.n_steps):
            for slot in range(R):
                chunk, kr, vr = opool.slots[(0, b, s, slot)]
                kg, vg = pool.fetch(0, b, s, slot)
                ek, ev = rel_err(host(kg), kr), rel_err(host(vg), vr)
                say(f"block {b} step {s} slot {slot} (chunk {chunk}): k err {ek:.2e}, v err {ev:.2e}")
                assert ek <= t and ev <= t


def test_schedule_groups_on_concurrent_streams_bitwise():
    """A tick's tasks split into two groups of steps on two HIP streams give
    bitwise the latents of one batch per block (1.3B width, 2 blocks, k = 2,
    6 chunks); and at the tiny fp32 shape they match the sequential oracle."""
    cfg = with_(C3, n_blocks=2)
    n_chunks = 6
    blocks, tw, ctxs, lat = _schedule_inputs(cfg, n_chunks, 1)
    say("schedule groups 1 vs 2, 1.3B width")
    a = _gpu_schedule(cfg, blocks, tw, ctxs, lat, n_chunks, 1, 2, groups=1)
    b = _gpu_schedule(cfg, blocks, tw, ctxs, lat, n_chunks, 1, 2, groups=2)
    assert np.array_equal(a, b) and np.all(np.isfinite(a))
    cfg = C1
    blocks, tw, ctxs, lat = _schedule_inputs(cfg, 4, 2)
    gx = _gpu_schedule(cfg, blocks, tw, ctxs, lat, 4, 2, 2, groups=2)
    ox, _ = oracle.run_schedule(cfg, blocks, tw, lambda sg, c: lat[(sg, c)], ctxs, 4, order="sequential")
    for c in range(4):
        for sg in range(2):
            e = rel_err(gx[c, sg], ox[(sg, c)])
            say(f"groups 2, chunk {c} stream {sg}: x^S err {e:.2e}")
            assert e <= 1e-4


@pytest.mark.parametrize("cfg", [C1, with_(C2, hidden=512, heads=8, head_dim=64, ffn=1024, n_ctx=200)],
                         ids=["tiny_fp32", "bf16_d64"])
def test_stage_step_replays_as_a_graph(cfg):
    """A stage batch and its Euler update captured into a HIP graph (on a
    stream an uncaptured call set up) and replayed three times, with eager
    work and synchronisations between the replays: every replay gives bitwise
    the eager call's output, latents and cache entries."""
    tasks = [(0, 5, 1, 2), (1, 4, 0, 2)]
    case = StageCase(cfg, tasks, n_slots=cfg.window + 2)
    ps_tasks = case.setup_gpu()
    h_in = to_dev(case.h_in, torch.float32)
    h_out = torch.empty_like(h_in)
    x0 = to_dev(inputs.hidden_rows(cfg, len(tasks), 0, tag="x0"), torch.float32)
    x = x0.clone()
    dts = [0.5, 0.25]
    stream = torch.cuda.Stream()
    say("graph replay", cfg.name)

    def step():
        runtime.stage_batch(case.pool, case.block, case.te, ps_tasks, h_in, h_out)
        runtime.euler_update(x, h_out, dts, cfg.tokens, cfg.hidden)

    with torch.cuda.stream(stream):
        step()
        x.copy_(x0)
        step()
    torch.cuda.synchronize()
    ref_h, ref_x = host(h_out), host(x)
    ref_kv = [host(t) for (sg, c, s_, _) in tasks for t in case.pool.fetch(sg, 0, s_, c % case.R)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        step()
    for rep in range(3):
        # eager work between replays: a plain call on other buffers
        other = torch.zeros_like(h_in)
        runtime.stage_batch(case.pool, case.block, case.te, ps_tasks, h_in, other)
        torch.cuda.synchronize()
        h_out.fill_(float("nan"))
        x.copy_(x0)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(h_out), ref_h), rep
        assert np.array_equal(host(x), ref_x), rep
        kv = [host(t) for (sg, c, s_, _) in tasks for t in case.pool.fetch(sg, 0, s_, c % case.R)]
        assert all(np.array_equal(a, b) for a, b in zip(kv, ref_kv)), rep


def test_capture_refuses_uncached_timestep_and_workspace_growth():
    """Under capture a call that would fill a timestep row or grow the
    stream's workspace is refused (PS_ERR_UNSUPPORTED) instead of enqueuing
    that work into the graph; the stream keeps working afterwards."""
    cfg = C1
    case = StageCase(cfg, [(0, 3, 1, 2), (0, 2, 1, 2)], n_slots=cfg.window + 2)
    ps_tasks = case.setup_gpu()
    L = cfg.tokens
    h = to_dev(case.h_in, torch.float32)
    one = h[:L]
    stream = torch.cuda.Stream()
    say("capture refusals")
    with torch.cuda.stream(stream):      # one task at step 1: workspace for one task, row t_1 cached
        runtime.stage_batch(case.pool, case.block, case.te, ps_tasks[1:], one, one)
    torch.cuda.synchronize()
    t0_task = runtime.make_task(0, 0, 0, cfg.timesteps[0], 0, [])   # step 0: its timestep is not cached
    for tasks, x, why in (([t0_task], one, "timestep"), (ps_tasks, h, "workspace")):
        graph = torch.cuda.CUDAGraph()
        with pytest.raises(PsError) as ei:
            with torch.cuda.graph(graph, stream=stream):
                runtime.stage_batch(case.pool, case.block, case.te, tasks, x, x)
        assert ei.value.status == _lib.PS_ERR_UNSUPPORTED and why in str(ei.value), str(ei.value)
        torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        runtime.stage_batch(case.pool, case.block, case.te, ps_tasks, h, h)
    torch.cuda.synchronize()
    assert torch.isfinite(h).all()


# ------------------------------------------------- patch embedding / head
@pytest.mark.parametrize("cfg", [C1, C3, C4], ids=lambda c: c.name)
def test_patch_embed_and_output_head(cfg):
    """Both steps either side of the block stack on one batch of tasks at
    different timesteps (the head's modulation differs per task)."""
    n = 3 if cfg is C1 else 2
    L, P, D = cfg.tokens, cfg.latent_dim, cfg.hidden
    hw = inputs.head_weights(cfg, 0)
    tw = inputs.time_weights(cfg, 0)
    x = np.concatenate([inputs.latent_patches(cfg, 0, c, 0) for c in range(n)])
    h = inputs.hidden_rows(cfg, n, 0, tag="head_h")
    ts = [cfg.timesteps[i % cfg.n_steps] for i in range(n)][::-1]
    say("head", cfg.name, "tasks", n, "timesteps", ts)
    td = runtime.ps_dtype(cfg.dtype)
    head = runtime.Head.from_numpy(hw, D, P, td)
    te = make_te(cfg, tw)
    xg = to_dev(x, torch.float32)
    h0 = torch.empty((n * L, D), dtype=torch.float32, device="cuda")
    runtime.patch_embed(head, xg, h0)
    v = torch.empty((n * L, P), dtype=torch.float32, device="cuda")
    runtime.output_head(head, te, ts, L, to_dev(h, torch.float32), v)
    torch.cuda.synchronize()
    e0 = rel_err(host(h0), oracle.patch_embed(x, hw))
    say(f"patch embed err {e0:.2e}")
    assert e0 <= tol(cfg)
    for i in range(n):
        ref = oracle.output_head(h[i * L:(i + 1) * L], oracle.time_mlp(ts[i], tw), hw)
        e = rel_err(host(v[i * L:(i + 1) * L]), ref)
        say(f"head task {i} (t = {ts[i]}) err {e:.2e}")
        assert e <= tol(cfg)


@pytest.mark.parametrize("k", [1, 2])
def test_schedule_c1_with_head_matches_oracle(k):
    """The tiny configuration end to end on latent patches: patch embedding,
    2 blocks x 2 steps, output head and Euler per tick (staggered on the GPU,
    sequential in the oracle)."""
    from autoregressive_denoising_dit_amd.schedule import StaggeredRunner
    cfg, n_chunks = C1, 4
    blocks, tw, ctxs, _ = _schedule_inputs(cfg, n_chunks, 1)
    hw = inputs.head_weights(cfg, 0)
    lat = {c: inputs.latent_patches(cfg, 0, c, 0) for c in range(n_chunks)}
    say("schedule c1 with head", k)
    pool = make_pool(cfg, n_streams=1, n_blocks=cfg.n_blocks, n_slots=cfg.window + k)
    blks = [make_block(cfg, w, b) for b, w in enumerate(blocks)]
    te = make_te(cfg, tw)
    for blk in blks:
        pool.context_set(blk, 0, to_dev(ctxs[0], torch.float32))
    head = runtime.Head.from_numpy(hw, cfg.hidden, cfg.latent_dim, runtime.ps_dtype(cfg.dtype))
    x = torch.stack([to_dev(lat[c], torch.float32)[None] for c in range(n_chunks)]).contiguous()
    StaggeredRunner(pool, blks, te, cfg.timesteps, cfg.window, k, 1, head=head).run(x, n_chunks)
    torch.cuda.synchronize()
    gx = host(x)
    ox, _ = oracle.run_schedule(cfg, blocks, tw, lambda sg, c: lat[c], ctxs, n_chunks, order="sequential",
                                head=hw)
    for c in range(n_chunks):
        e = rel_err(gx[c, 0], ox[(0, c)])
        say(f"chunk {c}: x^S err {e:.2e}")
        assert e <= 1e-4


def test_schedule_c1_shifted_timesteps_matches_oracle():
    """The tiny configuration end to end with a non-uniform (shift 3) schedule
    of three steps, on latent patches with the head."""
    from autoregressive_denoising_dit_amd.schedule import StaggeredRunner, shifted_timesteps
    ts = shifted_timesteps(3, 3.0)
    cfg, n_chunks, k = with_(C1, timesteps=ts), 4, 1
    blocks, tw, ctxs, _ = _schedule_inputs(cfg, n_chunks, 1)
    hw = inputs.head_weights(cfg, 0)
    lat = {c: inputs.latent_patches(cfg, 0, c, 0) for c in range(n_chunks)}
    say("schedule c1 shifted timesteps", ts)
    pool = make_pool(cfg, n_streams=1, n_blocks=cfg.n_blocks, n_slots=cfg.window + k)
    blks = [make_block(cfg, w, b) for b, w in enumerate(blocks)]
    te = make_te(cfg, tw)
    for blk in blks:
        pool.context_set(blk, 0, to_dev(ctxs[0], torch.float32))
    head = runtime.Head.from_numpy(hw, cfg.hidden, cfg.latent_dim, runtime.ps_dtype(cfg.dtype))
    x = torch.stack([to_dev(lat[c], torch.float32)[None] for c in range(n_chunks)]).contiguous()
    StaggeredRunner(pool, blks, te, ts, cfg.window, k, 1, head=head).run(x, n_chunks)
    torch.cuda.synchronize()
    gx = host(x)
    ocfg = with_(cfg, timesteps=oracle.shifted_timesteps(3, 3.0))
    ox, _ = oracle.run_schedule(ocfg, blocks, tw, lambda sg, c: lat[c], ctxs, n_chunks, order="sequential",
                                head=hw)
    for c in range(n_chunks):
        e = rel_err(gx[c, 0], ox[(0, c)])
        say(f"chunk {c}: x^S err {e:.2e}")
        assert e <= 1e-4


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_concurrent_batches_on_two_streams_match_sequential(name):
    """Two stage batches of disjoint pool regions, submitted on two HIP streams
    without synchronisation between them, give bitwise the outputs and cache
    entries of the same batches run one after the other on one stream."""
    cfg = {"c1": C1, "c2": C2}[name]
    W = cfg.window
    R = W + 1
    w = inputs.block_weights(cfg, 0, 0)
    tw = inputs.time_weights(cfg, 0)
    td = runtime.TORCH_DTYPE[runtime.ps_dtype(cfg.dtype)]
    n_per = 2 if name == "c1" else 1
    say("concurrent batches", name)

    def run(concurrent):
        pool = make_pool(cfg, n_streams=2 * n_per, n_blocks=1, n_slots=R, check_slots=False)
        blk = make_block(cfg, w, 0)
        te = make_te(cfg, tw)
        g = torch.Generator(device="cuda")
        g.manual_seed(5)
        shape = (cfg.tokens, cfg.heads, cfg.head_dim)
        for sg in range(2 * n_per):
            pool.context_set(blk, sg, (torch.randn(cfg.n_ctx, cfg.hidden, generator=g, device="cuda", dtype=torch.float32)).to(td))
            for st_ in range(cfg.n_steps):
                for slot in range(R):
                    pool.load(sg, 0, st_, slot, 0, torch.randn(*shape, generator=g, device="cuda", dtype=torch.float32).to(td),
                              torch.randn(*shape, generator=g, device="cuda", dtype=torch.float32).to(td))
        # batch A: streams 0..n_per-1; batch B: streams n_per..2 n_per-1; different steps
        c = W + 2
        mk = lambda sg, s: runtime.make_task(sg, c, s, cfg.timesteps[s], c % R, [(c - W + j) % R for j in range(W)])
        ta = [mk(sg, 0) for sg in range(n_per)]
        tb = [mk(n_per + sg, cfg.n_steps - 1) for sg in range(n_per)]
        xa = torch.randn(n_per * cfg.tokens, cfg.hidden, generator=g, device="cuda", dtype=torch.float32)
        xb = torch.randn(n_per * cfg.tokens, cfg.hidden, generator=g, device="cuda", dtype=torch.float32)
        ha, hb = torch.empty_like(xa), torch.empty_like(xb)
        # cache both timesteps first (a cache fill waits for the device)
        runtime.stage_batch(pool, blk, te, ta, xa, ha)
        runtime.stage_batch(pool, blk, te, tb, xb, hb)
        torch.cuda.synchronize()
        if concurrent:
            s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
            for _ in range(3):
                runtime.stage_batch(pool, blk, te, ta, xa, ha, cuda_stream=s1)
                runtime.stage_batch(pool, blk, te, tb, xb, hb, cuda_stream=s2)
        else:
            for _ in range(3):
                runtime.stage_batch(pool, blk, te, ta, xa, ha)
                runtime.stage_batch(pool, blk, te, tb, xb, hb)
        torch.cuda.synchronize()
        kv = [pool.fetch(sg, 0, s, c % R) for (sg, s) in
              [(i, 0) for i in range(n_per)] + [(n_per + i, cfg.n_steps - 1) for i in range(n_per)]]
        return host(ha), host(hb), [host(k) for k, _ in kv] + [host(v) for _, v in kv]

    seq, conc = run(False), run(True)
    np.testing.assert_array_equal(conc[0], seq[0])
    np.testing.assert_array_equal(conc[1], seq[1])
    for a, b in zip(conc[2], seq[2]):
        np.testing.assert_array_equal(a, b)


def test_head_rejects_bad_arguments():
    cfg = C3
    hw = {k: to_dev(v.T if v.ndim == 2 and k.startswith("w") else v,
                    torch.bfloat16 if k.startswith("w") else torch.float32)
          for k, v in inputs.head_weights(cfg, 0).items()}
    with pytest.raises(ValueError):
        runtime.Head(hw, cfg.hidden, cfg.latent_dim + 1, runtime.PS_BF16)
    bad = _lib.HeadDesc(cfg.hidden, 40, runtime.PS_BF16, *[hw[k].data_ptr() for k in
                                                          ("w_embed", "w_head", "b_embed", "b_head", "t_head")])
    h = ctypes.c_void_p()
    st = _lib.load().ps_head_create(ctypes.byref(bad), ctypes.byref(h))
    assert st == _lib.PS_ERR_INVALID_ARG
    head = runtime.Head(hw, cfg.hidden, cfg.latent_dim, runtime.PS_BF16)
    te = make_te(cfg, inputs.time_weights(cfg, 0))
    hh = torch.zeros((cfg.tokens, cfg.hidden), dtype=torch.float32, device="cuda")
    v = torch.zeros((cfg.tokens, cfg.latent_dim), dtype=torch.float32, device="cuda")
    with pytest.raises(_lib.PsError):
        runtime.output_head(head, te, [float("nan")], cfg.tokens, hh, v)


# ------------------------------------------------------------ error paths
def test_slot_ledger_rejects_stale_read():
    cfg = C1
    pool = make_pool(cfg, n_streams=1, n_blocks=1, check_slots=True)
    blk = make_block(cfg, inputs.block_weights(cfg, 0, 0))
    te = make_te(cfg, inputs.time_weights(cfg, 0))
    pool.context_set(blk, 0, to_dev(inputs.context(cfg, 0, 0), torch.float32))
    k, v = inputs.cache_entry(cfg, 0, 0, 0, 1, 0)
    pool.load(0, 0, 0, 1, 1, to_dev(k, torch.float32), to_dev(v, torch.float32))
    h = torch.zeros((cfg.tokens, cfg.hidden), dtype=torch.float32, device="cuda")
    # chunk 3 expects chunks 1, 2 in its read slots; slot 2 holds nothing
    bad = runtime.make_task(0, 3, 0, 1.0, 0, [1, 2])
    with pytest.raises(PsError) as ei:
        runtime.stage_batch(pool, blk, te, [bad], h, h)
    assert ei.value.status == PS_ERR_SLOT_CONFLICT
    # two tasks writing one slot
    t1 = runtime.make_task(0, 2, 0, 1.0, 0, [1])
    t2 = runtime.make_task(0, 2, 0, 1.0, 0, [1])
    h2 = torch.zeros((2 * cfg.tokens, cfg.hidden), dtype=torch.float32, device="cuda")
    with pytest.raises(PsError) as ei:
        runtime.stage_batch(pool, blk, te, [t1, t2], h2, h2)
    assert ei.value.status == PS_ERR_SLOT_CONFLICT
    # a valid call still works after the rejections
    ok = runtime.make_task(0, 2, 0, 1.0, 2, [1])
    runtime.stage_batch(pool, blk, te, [ok], h, h)
    torch.cuda.synchronize()
    assert torch.isfinite(h).all()


def test_pool_rejects_a_fifth_stream():
    """A pool keeps one workspace per HIP stream for up to four streams; a
    call on a fifth stream is refused before any launch, and the pool still
    works on the streams it knows."""
    cfg = C1
    pool = make_pool(cfg, n_streams=1, n_blocks=1, check_slots=False)
    blk = make_block(cfg, inputs.block_weights(cfg, 0, 0))
    te = make_te(cfg, inputs.time_weights(cfg, 0))
    pool.context_set(blk, 0, to_dev(inputs.context(cfg, 0, 0), torch.float32))
    h = torch.zeros((cfg.tokens, cfg.hidden), dtype=torch.float32, device="cuda")
    task = [runtime.make_task(0, 0, 0, 1.0, 0, [])]
    streams = [torch.cuda.Stream() for _ in range(5)]
    for st in streams[:4]:
        runtime.stage_batch(pool, blk, te, task, h, h, cuda_stream=st)
    torch.cuda.synchronize()
    with pytest.raises(PsError) as ei:
        runtime.stage_batch(pool, blk, te, task, h, h, cuda_stream=streams[4])
    assert ei.value.status == PS_ERR_INVALID_ARG and "streams" in str(ei.value)
    runtime.stage_batch(pool, blk, te, task, h, h, cuda_stream=streams[0])
    torch.cuda.synchronize()
    assert torch.isfinite(h).all()


def test_invalid_arguments_rejected():
    cfg = C1
    pool = make_pool(cfg, n_streams=1, n_blocks=1)
    blk = make_block(cfg, inputs.block_weights(cfg, 0, 0))
    te = make_te(cfg, inputs.time_weights(cfg, 0))
    h = torch.zeros((cfg.tokens, cfg.hidden), dtype=torch.float32, device="cuda")
    # context not set yet
    with pytest.raises(PsError) as ei:
        runtime.stage_batch(pool, blk, te, [runtime.make_task(0, 0, 0, 1.0, 0, [])], h, h)
    assert ei.value.status == PS_ERR_INVALID_ARG
    pool.context_set(blk, 0, to_dev(inputs.context(cfg, 0, 0), torch.float32))
    for bad in (runtime.make_task(1, 0, 0, 1.0, 0, []),       # stream out of range
                runtime.make_task(0, 0, 2, 1.0, 0, []),       # step out of range
                runtime.make_task(0, 0, 0, 1.0, 9, []),       # slot out of range
                runtime.make_task(0, 1, 0, 1.0, 0, [0]),      # reads its own write slot
                runtime.make_task(0, 0, 0, float("nan"), 0, [])):
        with pytest.raises(PsError) as ei:
            runtime.stage_batch(pool, blk, te, [bad], h, h)
        assert ei.value.status == PS_ERR_INVALID_ARG
