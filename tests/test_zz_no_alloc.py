"""ps_stage_batch_static (the stage call that allocates no device memory)
against ps_stage_batch on identical inputs: two calls in a row, the second
with a smaller batch, and a batch too large for its static workspace."""
import numpy as np
import pytest
import torch

from autoregressive_denoising_dit_amd import _lib, runtime
from synthetic import C1, C2
from tests.gpu_util import StageCase, make_block, make_pool, make_te, say, to_dev
from synthetic import inputs

pytestmark = pytest.mark.gpu


def _same(a, b):
    assert np.array_equal(a.gpu_h_out, b.gpu_h_out)
    assert a.gpu_kv.keys() == b.gpu_kv.keys()
    for key in a.gpu_kv:
        for x, y in zip(a.gpu_kv[key], b.gpu_kv[key]):
            assert np.array_equal(x, y)


@pytest.mark.parametrize("cfg", [C2, C1], ids=["w1536_bf16", "tiny_fp32"])
def test_static_workspace_matches_stage_batch(cfg):
    """Two tasks, then one (the second call smaller than the first, so the
    static workspace holds the first call's data in its tail): the outputs and
    the cache entries written equal ps_stage_batch's bit for bit."""
    S = cfg.n_steps
    first = [(0, 7, 2 % S, cfg.window), (1, 6, 1, cfg.window)]
    second = [(0, 5, S - 1, 2)]
    for tasks in (first, second):
        say("static workspace", cfg.name, tasks)
        plain = StageCase(cfg, tasks).run_gpu()
        stat = StageCase(cfg, tasks).run_gpu(static=True)
        _same(plain, stat)
        assert np.all(np.isfinite(stat.gpu_h_out))


def test_static_workspace_rejects_an_oversized_batch():
    """Four 1.3B-shaped tasks need about 170 MB of workspace, more than the
    128 MiB array: refused before anything is enqueued; the pool keeps working."""
    cfg = C2
    pool = make_pool(cfg, n_streams=4, n_blocks=1, check_slots=False)
    blk = make_block(cfg, inputs.block_weights(cfg, 0, 0))
    te = make_te(cfg, inputs.time_weights(cfg, 0))
    for sg in range(4):
        pool.context_set(blk, sg, to_dev(inputs.context(cfg, sg, 0), torch.bfloat16))
    tasks = [runtime.make_task(sg, 0, 0, 1.0, 0, []) for sg in range(4)]
    h = torch.zeros((4 * cfg.tokens, cfg.hidden), dtype=torch.float32, device="cuda")
    say("static workspace oversized")
    with pytest.raises(_lib.PsError) as ei:
        runtime.stage_batch_static(pool, blk, te, tasks, h, h)
    assert ei.value.status == _lib.PS_ERR_INVALID_ARG and "static" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.count_nonzero(h).item() == 0
    one = h[:cfg.tokens]
    runtime.stage_batch_static(pool, blk, te, tasks[:1], one, one)
    torch.cuda.synchronize()
    assert torch.isfinite(one).all() and torch.count_nonzero(one).item() > 0
