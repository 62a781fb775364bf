"""Shared set-up of the GPU parity tests: seeded inputs -> the HIP path through
the C ABI on one side, the float64 CPU oracle on the other."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from autoregressive_denoising_dit_amd import _lib, runtime
from synthetic import inputs

BF16_TOL = 3e-2    # max |err| / RMS(ref), bf16 operands
FP32_TOL = 1e-4    # max |err| / RMS(ref), fp32 operands


def tol(cfg):
    return BF16_TOL if cfg.dtype == "bf16" else FP32_TOL


def say(*a):
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite values from the GPU"
    rms = np.sqrt(np.mean(ref ** 2))
    return float(np.abs(got - ref).max() / rms)


def to_dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.float32))).to("cuda", dtype).contiguous()


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def make_pool(cfg, n_streams=None, n_blocks=None, n_slots=None, check_slots=True):
    return runtime.Pool(n_streams or cfg.n_streams, n_blocks or cfg.n_blocks, cfg.n_steps,
                        n_slots or cfg.ring, cfg.grid, cfg.heads, cfg.head_dim, cfg.n_ctx,
                        runtime.ps_dtype(cfg.dtype), check_slots=check_slots)


def make_block(cfg, w, block_index=0):
    return runtime.Block.from_numpy(w, cfg.hidden, cfg.heads, cfg.head_dim, cfg.ffn, block_index,
                                    runtime.ps_dtype(cfg.dtype))


def make_te(cfg, tw, capacity=16):
    return runtime.TimeEmbed.from_numpy(tw, cfg.hidden, capacity)


class StageCase:
    """One ps_stage_batch call on seeded inputs and its oracle counterpart.

    tasks: list of (stream, chunk, step, n_read).  The read slots of each task
    are pre-filled with seeded cache entries unless another task of the batch
    writes them (then the batch's own write is what is read)."""

    def __init__(self, cfg, tasks, seed=0, block_index=0, weights=None, tw=None, n_slots=None,
                 share_prefill=False):
        self.cfg, self.tasks, self.seed = cfg, tasks, seed
        self.w = weights if weights is not None else inputs.block_weights(cfg, block_index, seed)
        self.tw = tw if tw is not None else inputs.time_weights(cfg, seed)
        self.R = n_slots or max(cfg.ring, max(nr for (_, _, _, nr) in tasks) + 1)
        self.n_streams = max(t[0] for t in tasks) + 1
        self.td = runtime.TORCH_DTYPE[runtime.ps_dtype(cfg.dtype)]
        self.block_index = block_index
        written = {(sg, s, c) for (sg, c, s, _) in tasks}
        self.prefill = {}
        for (sg, c, s, nr) in tasks:
            for j in range(c - nr, c):
                if (sg, s, j) not in written and (sg, s, j) not in self.prefill:
                    if share_prefill:   # one seeded entry per (step, chunk), reused by every stream
                        src = next((v for (a, b, c2), v in self.prefill.items() if b == s and c2 == j), None)
                        self.prefill[(sg, s, j)] = src if src is not None else \
                            inputs.cache_entry(cfg, 0, block_index, s, j, seed)
                    else:
                        self.prefill[(sg, s, j)] = inputs.cache_entry(cfg, sg, block_index, s, j, seed)
        self.ctx = {sg: inputs.context(cfg, sg, seed) for sg in range(self.n_streams)}
        self.h_in = inputs.hidden_rows(cfg, len(tasks), seed)

    # ---------------------------------------------------------------- GPU
    def setup_gpu(self):
        """Pool (contexts set from the seeded tokens, window slots pre-filled),
        block and timestep embedding on the GPU; returns the batch's tasks."""
        cfg = self.cfg
        self.pool = make_pool(cfg, n_streams=self.n_streams, n_blocks=self.block_index + 1, n_slots=self.R)
        self.block = make_block(cfg, self.w, self.block_index)
        self.te = make_te(cfg, self.tw)
        for sg, ctx in self.ctx.items():
            self.pool.context_set(self.block, sg, to_dev(ctx, self.td))
        for (sg, s, j), (k, v) in self.prefill.items():
            self.pool.load(sg, self.block_index, s, j % self.R, j, to_dev(k, self.td), to_dev(v, self.td))
        self.ps_tasks = [runtime.make_task(sg, c, s, cfg.timesteps[s], c % self.R,
                                           [j % self.R for j in range(c - nr, c)])
                         for (sg, c, s, nr) in self.tasks]
        return self.ps_tasks

    def run_gpu(self, h_out_same=False, probe=False, static=False):
        cfg = self.cfg
        say("stage", cfg.name, "tasks", self.tasks)
        ps_tasks = self.setup_gpu()
        h_in = to_dev(self.h_in, torch.float32)
        h_out = h_in if h_out_same else torch.empty_like(h_in)
        if probe:
            M = len(self.tasks) * cfg.tokens
            self.gpu_probe = {
                name: torch.full((M, cfg.ffn if name == "u" else cfg.hidden), float("nan"), device="cuda",
                                 dtype=torch.float32 if name in _lib.PROBE_FP32 else self.td)
                for name in _lib.PROBE_FIELDS}
            runtime.stage_batch_probe(self.pool, self.block, self.te, ps_tasks, h_in, h_out, self.gpu_probe)
        elif static:
            runtime.stage_batch_static(self.pool, self.block, self.te, ps_tasks, h_in, h_out)
        else:
            runtime.stage_batch(self.pool, self.block, self.te, ps_tasks, h_in, h_out)
        torch.cuda.synchronize()
        self.gpu_h_out = host(h_out)
        self.gpu_kv = {}
        for (sg, c, s, nr) in self.tasks:
            k, v = self.pool.fetch(sg, self.block_index, s, c % self.R)
            self.gpu_kv[(sg, c, s)] = (host(k), host(v))
        torch.cuda.synchronize()
        return self

    # ------------------------------------------------------------- oracle
    def run_oracle(self, task_ids=None, rows=None):
        """Oracle h_out rows (all or a sample), cache entries of the tasks and
        each task's intermediates (self.ref_trace[i]: y1 and q over all rows,
        the rest over ``rows``)."""
        cfg, L = self.cfg, self.cfg.tokens
        ids = range(len(self.tasks)) if task_ids is None else task_ids
        E = {s: oracle.time_embedding(t, self.tw) for s, t in enumerate(cfg.timesteps)}
        ctx_kv = {}
        # the batch's own writes land before any read (a task may read what
        # another task of the batch writes); computed for the tasks needed
        own, own_trace = {}, {}
        where = {(sg, s, c): i for i, (sg, c, s, _) in enumerate(self.tasks)}

        def qkv(key):
            if key not in own:
                i = where[key]
                sg, c, s, _ = self.tasks[i]
                mod = oracle.modulation(E[s], self.w["tmod"])
                own_trace[key] = {}
                own[key] = oracle.qkv_phase(self.h_in[i * L:(i + 1) * L], mod, self.w, c, cfg.grid,
                                            cfg.heads, trace=own_trace[key])
            return own[key]

        out, self.ref_trace = {}, {}
        for i in ids:
            sg, c, s, nr = self.tasks[i]
            mod = oracle.modulation(E[s], self.w["tmod"])
            ent = []
            for j in range(c - nr, c):
                ent.append(qkv((sg, s, j))[1:] if (sg, s, j) in where else self.prefill[(sg, s, j)])
            q, k, v = qkv((sg, s, c))
            K = np.concatenate([e[0] for e in ent] + [k])
            V = np.concatenate([e[1] for e in ent] + [v])
            h = self.h_in[i * L:(i + 1) * L]
            if sg not in ctx_kv:
                ctx_kv[sg] = oracle.context_kv(self.ctx[sg], self.w, cfg.heads)
            tr = dict(own_trace[(sg, s, c)])
            out[i] = oracle.rest_phase(h, q, K, V, mod, self.w, *ctx_kv[sg], rows=rows, trace=tr)
            self.ref_trace[i] = tr
        self.ref_h_out = out
        self.ref_kv = {(sg, c, s): own[(sg, s, c)][1:] for (sg, c, s, _) in self.tasks if (sg, s, c) in own}
        return self
