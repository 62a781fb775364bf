"""Steps either side of the block stack, in float64 (oracle).

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's CPU
baseline may use this module; the product path never does.

The patch embedding turns a chunk's latent into the residual stream the first
block reads; the output head turns the last block's output into the velocity
the Euler step subtracts.  Sources: the pages evaluate Wan-family backbones
(AREX feed article on the PhysisServe report, section "实测数字") and cut the
latent video into chunks of one latent frame; a 60 x 104 latent frame in 2 x 2
patches is the 30 x 52 token grid of a chunk.  The pages print neither layer,
so both take the plainest Wan-style reading:

  * the latent of a chunk is carried patchified, x in R^{L x P} with
    P = C * pf * ph * pw (C latent channels, patch pf x ph x pw); token n is
    row-major over the token grid, and a patch vector is ordered
    (channel, frame offset, row offset, column offset);
  * patch embedding: h_0 = x W_e + b_e, W_e in R^{P x D} -- the same map as a
    3D convolution with kernel = stride = patch;
  * output head: (shift, scale) = u(t) + T_h with u(t) the D-wide output of
    the timestep MLP (before the 6-way projection of the blocks) and T_h in
    R^{2 x D}; v = (LN(h)(1 + scale) + shift) W_h + b_h, W_h in R^{D x P}.
"""
from __future__ import annotations

import numpy as np

from .block import F64, layer_norm, silu, sinusoid


def time_mlp(t, tw):
    """u(t) in R^D: SiLU(phi(t) Wt1 + bt1) Wt2 + bt2 -- the shared timestep MLP
    whose SiLU-projected output is e(t) (``time_embedding``)."""
    g = {k: np.asarray(v, dtype=F64) for k, v in tw.items()}
    return silu(sinusoid(t) @ g["wt1"] + g["bt1"]) @ g["wt2"] + g["bt2"]


def patchify(lat, patch):
    """[C, Fr, Hh, Ww] latent -> [L, P] patches (tokens row-major over the grid
    (Fr/pf, Hh/ph, Ww/pw); patch vector ordered (c, i, j, k))."""
    lat = np.asarray(lat)
    C, Fr, Hh, Ww = lat.shape
    pf, ph, pw = patch
    gf, gh, gw = Fr // pf, Hh // ph, Ww // pw
    out = np.empty((gf * gh * gw, C * pf * ph * pw), dtype=lat.dtype)
    n = 0
    for f in range(gf):
        for y in range(gh):
            for x in range(gw):
                blk = lat[:, f * pf:(f + 1) * pf, y * ph:(y + 1) * ph, x * pw:(x + 1) * pw]
                out[n] = blk.reshape(-1)
                n += 1
    return out


def unpatchify(xp, shape, patch):
    """Inverse of ``patchify``: [L, P] -> [C, Fr, Hh, Ww]."""
    C, Fr, Hh, Ww = shape
    pf, ph, pw = patch
    gf, gh, gw = Fr // pf, Hh // ph, Ww // pw
    lat = np.empty(shape, dtype=np.asarray(xp).dtype)
    n = 0
    for f in range(gf):
        for y in range(gh):
            for x in range(gw):
                lat[:, f * pf:(f + 1) * pf, y * ph:(y + 1) * ph, x * pw:(x + 1) * pw] = \
                    np.asarray(xp[n]).reshape(C, pf, ph, pw)
                n += 1
    return lat


def patch_embed(xp, hw):
    """h_0 = x W_e + b_e: [L, P] latent patches -> [L, D] residual stream."""
    return np.asarray(xp, dtype=F64) @ np.asarray(hw["w_embed"], dtype=F64) + np.asarray(hw["b_embed"], dtype=F64)


def output_head(h, u, hw):
    """v = (LN(h)(1 + scale) + shift) W_h + b_h with (shift, scale) = u + T_h."""
    m = np.asarray(hw["t_head"], dtype=F64) + np.asarray(u, dtype=F64)[None, :]
    y = layer_norm(h) * (1.0 + m[1]) + m[0]
    return y @ np.asarray(hw["w_head"], dtype=F64) + np.asarray(hw["b_head"], dtype=F64)
