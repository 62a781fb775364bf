"""Each kernel of the stage on identical inputs, against the oracle's matching
step (ps_stage_kernel through the C ABI).

The input of every kernel is the oracle's own intermediate of that point of the
block, rounded to the type the path stores it in (bf16 for the operands of the
GEMMs and attentions in bf16 workloads, fp32 for the residual stream); the
reference is the oracle's step applied to that same rounded input.  So each
comparison measures one kernel, not the rounding its inputs picked up on the
way.  Self-attention reads the window's cache entries: the prior chunks'
seeded entries and the oracle's own keys/values of the batch's chunks
(rounded), loaded into the pool.  Cross-attention reads the oracle's context
keys/values (rounded), loaded with ps_context_load.

Bar: max|err| / RMS(ref) <= 3e-2 in bf16, <= 1e-4 in fp32, on
every row of every checked task.  Two allowances, both the storage rounding of
the kernel's own output and nothing else: an output stored in bf16 (fp32) is
at most 2^-8 (2^-24) of its value away from the value it rounds, so that much
is taken off each element's error.  For the residual kernels the branch
delta (out - h_in) is checked as well, with the fp32 rounding of out.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from autoregressive_denoising_dit_amd import runtime
from synthetic import C1, C2, C3, C4, C5, inputs, with_
from tests.gpu_util import StageCase, host, rel_err, say, to_dev, tol

pytestmark = pytest.mark.gpu

STORE_ROUNDOFF = {"bf16": 2.0 ** -8, "fp32": 2.0 ** -24}


def _err(got, ref, u):
    """max(|got - ref| - u |ref|, 0) / RMS(ref)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite values from the GPU"
    return float(np.maximum(np.abs(got - ref) - u * np.abs(ref), 0.0).max() / np.sqrt(np.mean(ref ** 2)))


class KernelCase(StageCase):
    """A stage batch whose kernels are run one at a time on the oracle's
    intermediates.  ``check``: indices of the tasks whose rows are compared
    (every row); the other tasks of the batch get copies of a checked task's
    inputs so that the launch has the batch's full shape."""

    def __init__(self, cfg, tasks, check=None, **kw):
        super().__init__(cfg, tasks, **kw)
        self.check = list(range(len(tasks))) if check is None else list(check)

    def rb(self, a):
        """The value as the path stores a compute-dtype operand."""
        a = np.asarray(a, np.float32)
        return (inputs.round_bf16(a) if self.cfg.dtype == "bf16" else a).astype(np.float64)

    @staticmethod
    def f32(a):
        return np.asarray(a, np.float32).astype(np.float64)

    def oracle_chain(self):
        """Per task needed: the block's intermediates in float64 (exact chain)."""
        cfg, L, H = self.cfg, self.cfg.tokens, self.cfg.heads
        E = {s: oracle.time_embedding(t, self.tw) for s, t in enumerate(cfg.timesteps)}
        where = {(sg, s, c): i for i, (sg, c, s, _) in enumerate(self.tasks)}
        need = set(self.check)
        for i in self.check:   # same-batch writes a checked task reads
            sg, c, s, nr = self.tasks[i]
            need |= {where[(sg, s, j)] for j in range(c - nr, c) if (sg, s, j) in where}
        self.mod, self.qkv, self.chain = {}, {}, {}
        for i in sorted(need):
            sg, c, s, nr = self.tasks[i]
            mod = oracle.modulation(E[s], self.w["tmod"])
            self.mod[i] = mod
            y1 = oracle.adaln(self.h_in[i * L:(i + 1) * L], mod[0], mod[1])
            self.qkv[i] = oracle.qkv_proj(y1, self.w, c, cfg.grid, H) + (y1,)
        self.ctx_kv = {sg: oracle.context_kv(ctx, self.w, H) for sg, ctx in self.ctx.items()}
        for i in self.check:
            sg, c, s, nr = self.tasks[i]
            q, k, v, y1 = self.qkv[i]
            K, V = self.window(i, exact=True)
            tr = {"y1": y1}
            oracle.rest_phase(self.h_in[i * L:(i + 1) * L], q, K, V, self.mod[i], self.w, *self.ctx_kv[sg], trace=tr)
            self.chain[i] = tr
        return self

    def window(self, i, exact=False):
        """Keys/values task i attends to, oldest first: seeded prior entries or
        the batch's own (the oracle's keys/values, rounded unless ``exact``)."""
        sg, c, s, nr = self.tasks[i]
        where = {(a, b_, cc): j for j, (a, cc, b_, _) in enumerate(self.tasks)}
        ks, vs = [], []
        for j in list(range(c - nr, c)) + [c]:
            if (sg, s, j) in where:
                _, k, v, _ = self.qkv[where[(sg, s, j)]]
                if not exact:
                    k, v = self.rb(k), self.rb(v)
            else:
                k, v = self.prefill[(sg, s, j)]
            ks.append(k)
            vs.append(v)
        return np.concatenate(ks), np.concatenate(vs)

    def batch_input(self, per_task, cols):
        """[n L, cols] input: the checked tasks' rows, copies for the others."""
        L = self.cfg.tokens
        out = np.empty((len(self.tasks) * L, cols), np.float32)
        for i in range(len(self.tasks)):
            src = i if i in per_task else self.check[0]
            out[i * L:(i + 1) * L] = per_task[src]
        return out

    def run_kernel(self, name, x, fp_in, out_cols, fp_out, h_in=None):
        td = torch.float32 if fp_in else self.td
        xd = to_dev(x, td)
        out = torch.full((xd.shape[0], out_cols), float("nan"), device="cuda",
                         dtype=torch.float32 if fp_out else self.td)
        hd = to_dev(h_in, torch.float32) if h_in is not None else None
        runtime.stage_kernel(self.pool, self.block, self.te, self.ps_tasks, name, xd, out, hd)
        torch.cuda.synchronize()
        return host(out)


def _run_kernels(case):
    cfg, L, D, F, H, d = (case.cfg, case.cfg.tokens, case.cfg.hidden, case.cfg.ffn, case.cfg.heads,
                          case.cfg.head_dim)
    t, u_out = tol(cfg), STORE_ROUNDOFF[cfg.dtype]
    u32 = STORE_ROUNDOFF["fp32"]
    qscale = math.log2(math.e) / math.sqrt(d)
    case.setup_gpu()
    case.oracle_chain()
    rows = lambda a, i: a[i * L:(i + 1) * L]
    ch = case.chain
    worst = {}

    def score(name, got, refs, h_in=None, u=u_out):
        for i in case.check:
            g, r = rows(got, i), refs[i]
            e = _err(g, r, u)
            msg = f"{name} task {i} {case.tasks[i]}: err {e:.2e} (plain {rel_err(g, r):.2e})"
            if h_in is not None:
                hi = rows(h_in, i)
                ed = _err(g - hi, r - hi, 0.0) if cfg.dtype == "bf16" else \
                    float(np.maximum(np.abs((g - hi) - (r - hi)) - u32 * np.abs(r), 0).max()
                          / np.sqrt(np.mean((r - hi) ** 2)))
                msg += f", branch delta err {ed:.2e}"
                assert ed <= t, (name, i, ed)
            say(msg)
            worst[name] = max(worst.get(name, 0.0), e)
            assert e <= t, (name, i, e)

    # ln1: the residual stream as it is (fp32) -> y1
    got = case.run_kernel("ln1", case.h_in, True, D, False)
    score("ln1", got, {i: oracle.adaln(rows(case.h_in, i), case.mod[i][0], case.mod[i][1]) for i in case.check})

    # qkv: y1 (rounded) -> q (scaled), k / v into the write slot
    y1 = {i: case.rb(ch[i]["y1"]) for i in case.check}
    got = case.run_kernel("qkv", case.batch_input(y1, D), False, D, False)
    ref = {i: oracle.qkv_proj(y1[i], case.w, case.tasks[i][1], cfg.grid, H) for i in case.check}
    score("qkv q", got / qscale, {i: ref[i][0].reshape(L, D) for i in case.check})
    for i in case.check:
        sg, c, s, _ = case.tasks[i]
        k, v = case.pool.fetch(sg, case.block_index, s, c % case.R)
        for nm, g, r in (("k", host(k), ref[i][1]), ("v", host(v), ref[i][2])):
            e = _err(g, r, u_out)
            say(f"qkv {nm} task {i}: err {e:.2e}")
            assert e <= t, ("qkv " + nm, i, e)

    # self-attention: the oracle's q, k, v (rounded) in the window's slots
    for i in sorted(case.qkv):
        sg, c, s, _ = case.tasks[i]
        _, k, v, _ = case.qkv[i]
        case.pool.load(sg, case.block_index, s, c % case.R, c, to_dev(case.rb(k), case.td), to_dev(case.rb(v), case.td))
    qin = {i: case.rb(case.qkv[i][0].reshape(L, D) * qscale) for i in case.check}
    got = case.run_kernel("attn_self", case.batch_input(qin, D), False, D, False)
    ref = {}
    for i in case.check:
        K, V = case.window(i)
        ref[i] = oracle.attention((qin[i] / qscale).reshape(L, H, d), K, V).reshape(L, D)
    score("attn_self", got, ref)

    # O projection + gated residual
    a = {i: case.rb(ch[i]["attn"]) for i in case.check}
    h = case.h_in
    got = case.run_kernel("o_proj", case.batch_input(a, D), False, D, True, h_in=h)
    score("o_proj", got, {i: oracle.residual(rows(h, i), a[i], case.w["wo"], case.w["bo"], gate=case.mod[i][2])
                          for i in case.check}, h_in=h, u=u32)

    # ln2: h1 (fp32) -> y2
    h1 = {i: case.f32(ch[i]["h1"]) for i in case.check}
    got = case.run_kernel("ln2", case.batch_input(h1, D), True, D, False)
    score("ln2", got, {i: oracle.adaln(h1[i]) for i in case.check})

    # cross-attention queries
    y2 = {i: case.rb(ch[i]["y2"]) for i in case.check}
    got = case.run_kernel("xq_proj", case.batch_input(y2, D), False, D, False)
    score("xq_proj", got / qscale, {i: oracle.cross_q(y2[i], case.w, H).reshape(L, D) for i in case.check})

    # cross-attention over the oracle's context keys/values (rounded)
    for sg, (ck, cv) in case.ctx_kv.items():
        case.pool.context_load(sg, case.block_index, to_dev(case.rb(ck), case.td), to_dev(case.rb(cv), case.td))
    q2 = {i: case.rb(ch[i]["q2"] * qscale) for i in case.check}
    got = case.run_kernel("attn_cross", case.batch_input(q2, D), False, D, False)
    ref = {}
    for i in case.check:
        ck, cv = case.ctx_kv[case.tasks[i][0]]
        ref[i] = oracle.attention((q2[i] / qscale).reshape(L, H, d), case.rb(ck), case.rb(cv)).reshape(L, D)
    score("attn_cross", got, ref)

    # cross-O projection + residual
    xa = {i: case.rb(ch[i]["xattn"]) for i in case.check}
    h1b = case.batch_input(h1, D)
    got = case.run_kernel("xo_proj", case.batch_input(xa, D), False, D, True, h_in=h1b)
    score("xo_proj", got, {i: oracle.residual(h1[i], xa[i], case.w["wo2"], case.w["bo2"]) for i in case.check},
          h_in=h1b, u=u32)

    # ln3: h2 (fp32) -> y3
    h2 = {i: case.f32(ch[i]["h2"]) for i in case.check}
    got = case.run_kernel("ln3", case.batch_input(h2, D), True, D, False)
    score("ln3", got, {i: oracle.adaln(h2[i], case.mod[i][3], case.mod[i][4]) for i in case.check})

    # FFN1 + GELU-tanh
    y3 = {i: case.rb(ch[i]["y3"]) for i in case.check}
    got = case.run_kernel("ffn1", case.batch_input(y3, D), False, F, False)
    score("ffn1", got, {i: oracle.ffn_hidden(y3[i], case.w) for i in case.check})

    # FFN2 + gated residual
    uu = {i: case.rb(ch[i]["u"]) for i in case.check}
    h2b = case.batch_input(h2, D)
    got = case.run_kernel("ffn2", case.batch_input(uu, F), False, D, True, h_in=h2b)
    score("ffn2", got, {i: oracle.residual(h2[i], uu[i], case.w["w2"], case.w["b2"], gate=case.mod[i][5])
                        for i in case.check}, h_in=h2b, u=u32)
    say("worst per kernel:", {k: f"{v:.2e}" for k, v in worst.items()})


def _c3_batch():
    """Two chunks per step at all four steps (k = 2), the second of each pair
    reading the first one's same-batch write."""
    return [(0, 2 * (5 - s) + j, s, C3.window) for s in range(4) for j in range(2)]


def test_kernels_fp32_tiny():
    """fp32 workload: mixed chunks, steps and window fill, one task reading a
    same-batch write; every task, every row."""
    tasks = [(0, 0, 0, 0), (0, 3, 1, 2), (0, 2, 0, 2), (0, 4, 1, 2), (1, 1, 1, 1)]
    _run_kernels(KernelCase(C1, tasks, n_slots=8))


def test_kernels_bf16_head_dim_64_ragged_context():
    """64-dim heads at full chunk length (ragged last query and key tiles) and a
    200-token context (ragged last cross tile); both tasks, every row."""
    cfg = with_(C2, hidden=512, heads=8, head_dim=64, ffn=1024, n_ctx=200)
    _run_kernels(KernelCase(cfg, [(0, 5, 1, 3), (1, 4, 2, 2)]))


def test_kernels_c2_wan13b_single_task():
    """The 1.3B shape at batch 1, full window, every row."""
    _run_kernels(KernelCase(C2, [(0, 7, 2, 3)]))


def test_kernels_c3_wan13b_batch_of_eight():
    """The 1.3B time-shared batch of 8 mixed-step tasks; all 8 tasks, every row."""
    _run_kernels(KernelCase(C3, _c3_batch(), n_slots=C3.window + 2))


def test_kernels_c4_wan22_5b():
    """The 5B shape (1760-token chunks: ragged last query and key tiles, 24
    heads); both tasks, every row."""
    _run_kernels(KernelCase(C4, [(0, 9, 3, 3), (0, 12, 0, 3)]))


def test_kernels_c5_wan14b_sixteen_streams():
    """The 16-task 14B batch the benchmark times (16 streams at mixed steps);
    one task per denoising step checked, every row."""
    tasks = [(i, 10 + i // 4, (i * 3) % 4, 3) for i in range(16)]
    _run_kernels(KernelCase(C5, tasks, check=[0, 1, 2, 3], share_prefill=True))
