"""Pins of the oracle's patch embedding, output head and the schedules that
use them (no GPU).

Patch embedding: the same map as a 3D convolution whose kernel and stride are
the patch (torch's conv3d, float64 on the CPU), which also fixes the token and
patch-vector order.  Output head: torch's layer_norm and linear composed, plus
special cases with closed forms.  Schedules: staggered == sequential bitwise
with the head as without it, and a constant-velocity head gives the Euler
closed form."""
import numpy as np
import pytest
import torch

import oracle
from synthetic import C1, inputs, with_

torch.set_default_dtype(torch.float64)


def _tiny(**kw):
    base = dict(hidden=32, heads=2, head_dim=16, ffn=48, grid=(1, 2, 4), n_ctx=4, latent_channels=3,
                patch=(1, 2, 2))
    base.update(kw)
    return with_(C1, **base)


def test_patchify_hand_example_and_round_trip():
    lat = np.arange(2 * 1 * 2 * 4, dtype=np.float64).reshape(2, 1, 2, 4)   # C=2, 1 x 2 x 4 latent
    xp = oracle.patchify(lat, (1, 2, 2))
    assert xp.shape == (2, 8)                 # 1 x 1 x 2 tokens, P = 2 * 1 * 2 * 2
    # token 1 covers columns 2..3; vector order (channel, frame, row, col)
    np.testing.assert_array_equal(xp[1], [2, 3, 6, 7, 10, 11, 14, 15])
    rng = np.random.default_rng(0)
    big = rng.standard_normal((3, 2, 6, 8))
    xp2 = oracle.patchify(big, (2, 3, 2))
    np.testing.assert_array_equal(oracle.unpatchify(xp2, big.shape, (2, 3, 2)), big)


@pytest.mark.parametrize("patch", [(1, 2, 2), (2, 1, 2)])
def test_patch_embed_is_strided_conv3d(patch):
    rng = np.random.default_rng(1)
    C, D = 3, 10
    pf, ph, pw = patch
    lat = rng.standard_normal((C, 2 * pf, 3 * ph, 2 * pw))
    P = C * pf * ph * pw
    hw = {"w_embed": rng.standard_normal((P, D)), "b_embed": rng.standard_normal(D)}
    h = oracle.patch_embed(oracle.patchify(lat, patch), hw)
    wconv = torch.tensor(hw["w_embed"].T.reshape(D, C, pf, ph, pw))
    ref = torch.nn.functional.conv3d(torch.tensor(lat)[None], wconv, torch.tensor(hw["b_embed"]), stride=patch)
    ref = ref[0].permute(1, 2, 3, 0).reshape(-1, D).numpy()   # tokens row-major over (f, y, x)
    np.testing.assert_allclose(h, ref, rtol=1e-12, atol=1e-12)


def test_output_head_library_composition_and_special_cases():
    rng = np.random.default_rng(2)
    L, D, P = 7, 16, 12
    h = rng.standard_normal((L, D)) * 3 + 1
    u = rng.standard_normal(D)
    hw = {"w_head": rng.standard_normal((D, P)), "b_head": rng.standard_normal(P),
          "t_head": rng.standard_normal((2, D))}
    v = oracle.output_head(h, u, hw)
    th = torch.tensor
    shift, scale = th(hw["t_head"][0] + u), th(hw["t_head"][1] + u)
    y = torch.nn.functional.layer_norm(th(h), (D,), eps=1e-6) * (1 + scale) + shift
    ref = torch.nn.functional.linear(y, th(hw["w_head"].T), th(hw["b_head"])).numpy()
    np.testing.assert_allclose(v, ref, rtol=1e-12, atol=1e-12)
    # T_h = -u: no modulation, v = LN(h) W + b
    hw0 = dict(hw, t_head=np.stack([-u, -u]))
    ln = torch.nn.functional.layer_norm(th(h), (D,), eps=1e-6).numpy()
    np.testing.assert_allclose(oracle.output_head(h, u, hw0), ln @ hw["w_head"] + hw["b_head"], rtol=1e-12,
                               atol=1e-12)
    # zero head weights: v is the bias, exactly
    hwz = dict(hw, w_head=np.zeros((D, P)))
    np.testing.assert_array_equal(oracle.output_head(h, u, hwz), np.broadcast_to(hw["b_head"], (L, P)))


def test_time_mlp_feeds_the_time_embedding():
    cfg = _tiny()
    tw = inputs.time_weights(cfg, 0)
    for t in (1.0, 0.25):
        u = oracle.time_mlp(t, tw)
        e = oracle.silu(u) @ tw["wp"].astype(np.float64) + tw["bp"].astype(np.float64)
        np.testing.assert_allclose(e.reshape(6, -1), oracle.time_embedding(t, tw), rtol=1e-13, atol=1e-13)


def _run(cfg, n_chunks, order, k=1, n_streams=1, head=None, n_slots=None, blocks=None):
    if blocks is None:
        blocks = [{kk: v * 8.0 for kk, v in inputs.block_weights(cfg, b, 0).items()} for b in range(cfg.n_blocks)]
    tw = inputs.time_weights(cfg, 0)
    ctxs = [inputs.context(cfg, sg, 0) for sg in range(n_streams)]
    return oracle.run_schedule(cfg, blocks, tw, lambda sg, c: inputs.latent_patches(cfg, sg, c, 0), ctxs,
                               n_chunks, order=order, k=k, n_slots=n_slots,
                               head=head if head is not None else inputs.head_weights(cfg, 0))


@pytest.mark.parametrize("k,n_streams", [(1, 1), (2, 1), (2, 2)])
def test_staggered_equals_sequential_bitwise_with_head(k, n_streams):
    cfg = _tiny()
    R = cfg.window + 2
    xs, _ = _run(cfg, 5, "sequential", n_streams=n_streams, n_slots=R)
    xt, _ = _run(cfg, 5, "staggered", k=k, n_streams=n_streams, n_slots=R)
    assert xs.keys() == xt.keys()
    for key in xs:
        assert xs[key].shape == (cfg.tokens, cfg.latent_dim)
        assert xs[key].tobytes() == xt[key].tobytes(), key


def test_euler_closed_form_constant_velocity_head():
    """A head with zero weights predicts v = b_h for every token and step, so
    x^S = x^0 - (t_0 - t_S) b_h = x^0 - t_0 b_h (dyadic values: exact)."""
    cfg = _tiny(n_blocks=2, timesteps=(1.0, 0.5))
    hw = {k: v.astype(np.float64) for k, v in inputs.head_weights(cfg, 0).items()}
    hw["w_head"][:] = 0
    hw["b_head"] = np.arange(cfg.latent_dim) / 8.0
    x, _ = _run(cfg, 3, "staggered", head=hw)
    for c in range(3):
        x0 = inputs.latent_patches(cfg, 0, c, 0).astype(np.float64)
        np.testing.assert_array_equal(x[(0, c)], x0 - 0.5 * hw["b_head"] - 0.5 * hw["b_head"])


def test_head_uses_the_step_timestep_identity_blocks():
    """With identity blocks (zero gates, zero cross branch) a chunk's latent
    follows x <- x - (t_s - t_{s+1}) head(embed(x), u(t_s)) step by step; the
    schedule must reproduce that plain Euler loop, which pins that step s uses
    u(t_s) (the steps' timesteps differ, so any other pairing shows)."""
    cfg = _tiny(n_blocks=2, timesteps=(1.0, 0.75, 0.5, 0.25))
    tw = {k: v.astype(np.float64).copy() for k, v in inputs.time_weights(cfg, 0).items()}
    D = cfg.hidden
    blocks = []
    for b in range(cfg.n_blocks):
        w = {k: v.astype(np.float64) for k, v in inputs.block_weights(cfg, b, 0).items()}
        w["wo2"][:] = 0
        w["bo2"][:] = 0
        blocks.append(w)
    for row in (2, 5):
        tw["wp"][:, row * D:(row + 1) * D] = 0
        tw["bp"][row * D:(row + 1) * D] = 0
        for w in blocks:
            w["tmod"][row] = 0
    hw = {k: v.astype(np.float64) * 20.0 for k, v in inputs.head_weights(cfg, 0).items()}
    ctxs = [inputs.context(cfg, 0, 0)]
    x, _ = oracle.run_schedule(cfg, blocks, tw, lambda sg, c: inputs.latent_patches(cfg, sg, c, 0), ctxs, 2,
                               order="staggered", head=hw)
    ts = list(cfg.timesteps) + [0.0]
    for c in range(2):
        xr = inputs.latent_patches(cfg, 0, c, 0).astype(np.float64)
        for s in range(cfg.n_steps):
            v = oracle.output_head(oracle.patch_embed(xr, hw), oracle.time_mlp(ts[s], tw), hw)
            xr = xr - (ts[s] - ts[s + 1]) * v
        np.testing.assert_allclose(x[(0, c)], xr, rtol=1e-12, atol=1e-12)
