"""Pins of the oracle's chunk x step schedules (no GPU).

The method's claim is that staggering chunks and batching tasks of different
chunks and steps change nothing numerically; the oracle must therefore give
bitwise identical results under both schedules.  Causality, the window and the
ring discipline are checked on tiny runs."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle.schedule import SlotConflict
from synthetic import C1, inputs, with_

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bump(cfg):
    """A non-constant perturbation (a constant shift of a row is invisible
    through LayerNorm, so it would hide a dependence)."""
    return np.random.default_rng(99).standard_normal((cfg.tokens, cfg.hidden))


def _tiny(**kw):
    base = dict(hidden=32, heads=2, head_dim=16, ffn=48, grid=(1, 2, 4), n_ctx=4)
    base.update(kw)
    return with_(C1, **base)


def _run(cfg, n_chunks, order, k=1, n_streams=1, latent=None, n_slots=None, seed=0):
    blocks = [inputs.block_weights(cfg, b, seed) for b in range(cfg.n_blocks)]
    # stronger weights than the workloads so chunks visibly influence each other
    blocks = [{kk: v * 8.0 for kk, v in w.items()} for w in blocks]
    tw = inputs.time_weights(cfg, seed)
    ctxs = [inputs.context(cfg, sg, seed) for sg in range(n_streams)]
    lat = latent or (lambda sg, c: inputs.latent(cfg, sg, c, seed))
    return oracle.run_schedule(cfg, blocks, tw, lat, ctxs, n_chunks, order=order, k=k,
                               n_slots=n_slots)


def _same_bits(xa, xb):
    assert xa.keys() == xb.keys()
    for key in xa:
        assert xa[key].tobytes() == xb[key].tobytes(), key


@pytest.mark.parametrize("k,n_streams", [(1, 1), (2, 1), (1, 2), (2, 2)])
def test_staggered_equals_sequential_bitwise(k, n_streams):
    cfg = _tiny()
    R = cfg.window + 2
    xs, ps = _run(cfg, 5, "sequential", n_streams=n_streams, n_slots=R)
    xt, pt = _run(cfg, 5, "staggered", k=k, n_streams=n_streams, n_slots=R)
    _same_bits(xs, xt)
    assert ps.slots.keys() == pt.slots.keys()
    for key in ps.slots:
        a, b = ps.slots[key], pt.slots[key]
        assert a[0] == b[0]
        assert a[1].tobytes() == b[1].tobytes() and a[2].tobytes() == b[2].tobytes()


def test_deterministic():
    cfg = _tiny()
    xa, _ = _run(cfg, 3, "staggered", k=2)
    xb, _ = _run(cfg, 3, "staggered", k=2)
    _same_bits(xa, xb)


def test_causality():
    """Changing chunk 3's noise leaves chunks 0..2 unchanged and changes chunk 3, 4."""
    cfg = _tiny()
    base = lambda sg, c: inputs.latent(cfg, sg, c, 0)
    pert = lambda sg, c: base(sg, c) + (_bump(cfg) if c == 3 else 0.0)
    xa, _ = _run(cfg, 5, "staggered", k=1, latent=base)
    xb, _ = _run(cfg, 5, "staggered", k=1, latent=pert)
    for c in range(3):
        assert xa[(0, c)].tobytes() == xb[(0, c)].tobytes()
    for c in (3, 4):
        assert np.abs(xa[(0, c)] - xb[(0, c)]).max() > 1e-6


def test_window_is_strict_for_one_block_one_step():
    """With one block and one step a chunk sees exactly W earlier chunks."""
    cfg = _tiny(n_blocks=1, timesteps=(1.0,), window=2)
    base = lambda sg, c: inputs.latent(cfg, sg, c, 0)
    pert = lambda sg, c: base(sg, c) + (_bump(cfg) if c == 1 else 0.0)
    xa, _ = _run(cfg, 5, "sequential", latent=base)
    xb, _ = _run(cfg, 5, "sequential", latent=pert)
    assert xa[(0, 4)].tobytes() == xb[(0, 4)].tobytes()      # 4 - 1 > W
    assert np.abs(xa[(0, 3)] - xb[(0, 3)]).max() > 1e-6       # 3 - 1 <= W


def test_zero_window_chunks_independent():
    cfg = _tiny(window=0)
    base = lambda sg, c: inputs.latent(cfg, sg, c, 0)
    pert = lambda sg, c: base(sg, c) + (_bump(cfg) if c == 0 else 0.0)
    xa, _ = _run(cfg, 3, "staggered", latent=base)
    xb, _ = _run(cfg, 3, "staggered", latent=pert)
    for c in (1, 2):
        assert xa[(0, c)].tobytes() == xb[(0, c)].tobytes()


def test_streams_independent():
    cfg = _tiny()
    base = lambda sg, c: inputs.latent(cfg, sg, c, 0)
    pert = lambda sg, c: base(sg, c) + (_bump(cfg) if sg == 1 else 0.0)
    xa, _ = _run(cfg, 3, "staggered", n_streams=2, latent=base)
    xb, _ = _run(cfg, 3, "staggered", n_streams=2, latent=pert)
    for c in range(3):
        assert xa[(0, c)].tobytes() == xb[(0, c)].tobytes()


def test_ring_too_small_is_detected():
    """R = W + k is the smallest ring the staggered schedule can use; one less
    clobbers a live entry and the ledger says so."""
    cfg = _tiny()
    _run(cfg, 5, "staggered", k=2, n_slots=cfg.window + 2)
    with pytest.raises(SlotConflict):
        _run(cfg, 5, "staggered", k=2, n_slots=cfg.window + 1)


def test_euler_closed_form_identity_block():
    """With zero gates and a zero cross branch every block is the identity, so
    v = x^s and x^{s+1} = (1 - (t_s - t_{s+1})) x^s; over t = (1, 0.5) and t_S = 0
    that is x^S = 0.5 * 0.5 * x^0."""
    cfg = _tiny(n_blocks=2, timesteps=(1.0, 0.5))
    tw = inputs.time_weights(cfg, 0)
    E = [oracle.time_embedding(t, tw) for t in cfg.timesteps]
    blocks = []
    for b in range(cfg.n_blocks):
        w = {k: v.astype(np.float64) for k, v in inputs.block_weights(cfg, b, 0).items()}
        w["wo2"][:] = 0
        w["bo2"][:] = 0
        blocks.append(w)
    # gates are e(t)[2] + T[2] and e(t)[5] + T[5]: zero them for both timesteps by
    # giving the shared embedding zero output rows 2 and 5
    tw = {k: v.astype(np.float64).copy() for k, v in tw.items()}
    D = cfg.hidden
    for row in (2, 5):
        tw["wp"][:, row * D:(row + 1) * D] = 0
        tw["bp"][row * D:(row + 1) * D] = 0
        for w in blocks:
            w["tmod"][row] = 0
    x0 = {c: inputs.latent(cfg, 0, c, 0).astype(np.float64) for c in range(3)}
    x, _ = oracle.run_schedule(cfg, blocks, tw, lambda sg, c: x0[c],
                               [inputs.context(cfg, 0, 0)], 3, order="staggered")
    for c in range(3):
        np.testing.assert_array_equal(x[(0, c)], 0.25 * x0[c])
    del E


def test_fig2_stage_path_and_steady_output():
    """The pages' 2-step x 4-block example: chunk 7 passes the 8 stages in
    step-major order, and once the pipeline is full one chunk finishes per tick."""
    g = json.load(open(os.path.join(GOLDEN, "fig2_stage_pipeline.json")))
    S, B, c7 = g["n_steps"], g["n_blocks"], g["chunk"]
    assert S * B == g["n_stages"]
    ticks = oracle.staggered_ticks(12, S, 1)
    path = []
    for tasks in ticks:
        for b in range(B):
            path += [[s, b] for (_, c, s) in tasks if c == c7]
    assert path == g["stage_path_of_chunk"]
    done = [sum(1 for (_, c, s) in tasks if s == S - 1) for tasks in ticks]
    fill = S - 1
    assert all(n == g["completions_per_interval_after_fill"] for n in done[fill:])
    assert all(n == 0 for n in done[:fill])


@pytest.mark.parametrize("k", [1, 2, 3])
def test_staggered_ticks_cover_each_task_once(k):
    S, N = 4, 24
    ticks = oracle.staggered_ticks(N, S, k, 2)
    seen = [t for tasks in ticks for t in tasks]
    assert sorted(seen) == sorted((sg, c, s) for sg in range(2) for c in range(N) for s in range(S))
    # a chunk's steps come in order on consecutive ticks
    when = {t: i for i, tasks in enumerate(ticks) for t in tasks}
    for c in range(N):
        for s in range(1, S):
            assert when[(0, c, s)] == when[(0, c, s - 1)] + 1
    # steady state: k tasks per step per stream
    mid = ticks[S + 1]
    assert len(mid) == 2 * S * k


# --- non-uniform timestep schedules -------------------------------------------
def test_shifted_timesteps_special_cases():
    # shift 1 is the uniform grid the configs use
    assert oracle.shifted_timesteps(4, 1.0) == pytest.approx((1.0, 0.75, 0.5, 0.25), abs=0)
    # hand values: shift 3 maps u = 0.5 to 1.5 / 2 = 0.75 and u = 0.25 to 0.75 / 1.5 = 0.5
    t = oracle.shifted_timesteps(4, 3.0)
    assert t[0] == 1.0 and t[2] == pytest.approx(0.75, rel=1e-15) and t[3] == pytest.approx(0.5, rel=1e-15)
    assert oracle.shifted_timesteps(1, 5.0) == (1.0,)


@pytest.mark.parametrize("shift", [0.5, 1.0, 3.0, 5.0])
def test_shifted_timesteps_invert_to_the_uniform_grid(shift):
    S = 7
    t = np.array(oracle.shifted_timesteps(S, shift))
    assert np.all(np.diff(t) < 0) and t[0] == 1.0 and t[-1] > 0
    # the warp's inverse u = t / (a - (a - 1) t) recovers 1 - s/S
    u = t / (shift - (shift - 1.0) * t)
    np.testing.assert_allclose(u, 1.0 - np.arange(S) / S, rtol=1e-14)
    # a > 1 keeps every step at or above the uniform one (more time at high noise)
    if shift > 1:
        assert np.all(t >= 1.0 - np.arange(S) / S)


def test_shifted_timesteps_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.shifted_timesteps(0, 1.0)
    with pytest.raises(ValueError):
        oracle.shifted_timesteps(4, 0.0)
