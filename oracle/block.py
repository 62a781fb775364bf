"""One DiT block at one denoising step for one chunk, in float64 (oracle).

Sources.  The pages (PhysisServe tech-report summaries) define the unit of work
but print no formulas:
  * a stage is one Transformer block at one denoising step
    (AREX feed article, section "三层设计", layer 1; 163.com release, section
    "PhysisServe", bullet "Stage-wise 流水线");
  * chunk c at step s reads the still-noisy KV cache that the earlier chunk left
    at that same step (AREX article, section "难题"; 163.com release, section
    "新一代物理 AI 的基础设施", Fig. 1);
  * the blocks are 3D spatio-temporal attention blocks of Wan-family video DiTs
    (aicoder news, "Background and the Problem"; AREX article, "实测数字").
The block internals therefore take the plainest reading of a Wan-style DiT
block: AdaLN-modulated self-attention with 3D RoPE and a gate, cross-attention
to conditioning tokens, and an AdaLN-modulated GELU-tanh FFN with a gate, with
6-way modulation from a timestep embedding.  Each function's docstring
states the reading it takes.

Everything here is float64 and processes one task at a time.  Tensors:
h [L, D] residual stream; q, k, v [L, H, d]; weights [in, out] (y = x @ W + b).
"""
from __future__ import annotations

import numpy as np

F64 = np.float64
LN_EPS = 1e-6
ROPE_BASE = 10000.0
FREQ_DIM = 256
TIME_SCALE = 1000.0


def silu(z):
    """SiLU(z) = z * sigmoid(z)."""
    return z / (1.0 + np.exp(-z))


def gelu_tanh(z):
    """GELU with the tanh approximation: z/2 * (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3)))."""
    return 0.5 * z * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (z + 0.044715 * z ** 3)))


def layer_norm(z):
    """Row LayerNorm without affine: (z - mean) / sqrt(biased var + 1e-6)."""
    z = np.asarray(z, dtype=F64)
    mu = z.mean(axis=-1, keepdims=True)
    var = ((z - mu) ** 2).mean(axis=-1, keepdims=True)
    return (z - mu) / np.sqrt(var + LN_EPS)


def sinusoid(t):
    """256 sinusoidal features of a timestep: [cos(1000 t w_j) | sin(1000 t w_j)],
    w_j = 10000^(-j/128), j = 0..127."""
    half = FREQ_DIM // 2
    w = ROPE_BASE ** (-np.arange(half, dtype=F64) / half)
    a = TIME_SCALE * F64(t) * w
    return np.concatenate([np.cos(a), np.sin(a)])


def time_embedding(t, tw):
    """e(t) in R^{6 x D}: SiLU(SiLU(phi(t) Wt1 + bt1) Wt2 + bt2) Wp + bp.

    One shared timestep MLP and one shared D -> 6D projection for all blocks;
    the per-block part is the additive table added in ``modulation``."""
    g = {k: np.asarray(v, dtype=F64) for k, v in tw.items()}
    u = silu(sinusoid(t) @ g["wt1"] + g["bt1"]) @ g["wt2"] + g["bt2"]
    e = silu(u) @ g["wp"] + g["bp"]
    return e.reshape(6, -1)


def modulation(e, tmod):
    """m_b(t) = e(t) + T_b, rows (shift1, scale1, gate1, shift2, scale2, gate2)."""
    return np.asarray(e, dtype=F64) + np.asarray(tmod, dtype=F64)


def rope_segments(d):
    """Head-dim split of 3D RoPE into (frame, row, col) segments:
    (d - 4*floor(d/6), 2*floor(d/6), 2*floor(d/6))."""
    s = d // 6
    return (d - 4 * s, 2 * s, 2 * s)


def token_positions(chunk, grid):
    """[L, 3] integer (frame, row, col) of each token of a chunk.

    Token n is row-major over the chunk's latent grid (F_c, H_g, W_g):
    n = (f_loc * H_g + y) * W_g + x, and its frame is chunk * F_c + f_loc."""
    fc, hg, wg = grid
    pos = np.zeros((fc * hg * wg, 3), dtype=np.int64)
    n = 0
    for f in range(fc):
        for y in range(hg):
            for x in range(wg):
                pos[n] = (chunk * fc + f, y, x)
                n += 1
    return pos


def rope3d(x, pos):
    """Rotate each adjacent pair (2i, 2i+1) of every segment by angle p * theta_i,
    theta_i = 10000^(-2i/d_a), p the token's coordinate on that segment's axis.

    x: [L, H, d]; pos: [L, 3].  (u, w) -> (u cos - w sin, u sin + w cos)."""
    x = np.asarray(x, dtype=F64)
    out = x.copy()
    d = x.shape[-1]
    off = 0
    for axis, da in enumerate(rope_segments(d)):
        p = pos[:, axis].astype(F64)
        for i in range(da // 2):
            theta = ROPE_BASE ** (-2.0 * i / da)
            ang = p * theta
            c = np.cos(ang)[:, None]
            s = np.sin(ang)[:, None]
            u = x[:, :, off + 2 * i]
            w = x[:, :, off + 2 * i + 1]
            out[:, :, off + 2 * i] = u * c - w * s
            out[:, :, off + 2 * i + 1] = u * s + w * c
        off += da
    return out


def attention(q, k, v):
    """Per head: softmax(q k^T / sqrt(d)) v, max-subtracted.  No mask.

    q: [Lq, H, d]; k, v: [Lk, H, d] -> [Lq, H, d]."""
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    d = q.shape[-1]
    out = np.empty_like(q)
    for h in range(q.shape[1]):
        s = q[:, h, :] @ k[:, h, :].T / np.sqrt(d)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, h, :]
    return out


def _lin(x, w, b):
    return x @ np.asarray(w, dtype=F64) + np.asarray(b, dtype=F64)


def context_kv(ctx, w, heads):
    """Cross-attention keys/values of the conditioning tokens: [Lc, H, d] each.
    Depends only on (stream, block), so it may be computed once and reused."""
    ctx = np.asarray(ctx, dtype=F64)
    D = ctx.shape[1]
    kv = _lin(ctx, w["wkv2"], w["bkv2"])
    return kv[:, :D].reshape(-1, heads, D // heads), kv[:, D:].reshape(-1, heads, D // heads)


def adaln(h, shift=None, scale=None):
    """The block's normalisation step: LN(h)(1 + scale) + shift, or plain LN(h)
    without modulation (the cross-attention pre-norm).  [L, D] -> [L, D]."""
    y = layer_norm(h)
    if scale is None:
        return y
    return y * (1.0 + scale) + shift


def qkv_proj(y, w, chunk, grid, heads):
    """Queries, keys and values of the self-attention: y Wqkv + bqkv split into
    (q | k | v), then RoPE3D on q and k at the chunk's token positions.
    y [L, D] -> q, k, v [L, H, d]; (k, v) is the chunk's noisy-KV cache entry."""
    y = np.asarray(y, dtype=F64)
    L, D = y.shape
    d = D // heads
    qkv = _lin(y, w["wqkv"], w["bqkv"])
    q = qkv[:, :D].reshape(L, heads, d)
    k = qkv[:, D:2 * D].reshape(L, heads, d)
    v = qkv[:, 2 * D:].reshape(L, heads, d)
    pos = token_positions(chunk, grid)
    return rope3d(q, pos), rope3d(k, pos), v


def residual(h, x, wmat, bias, gate=None):
    """The residual update after a branch: h + gate * (x W + b), or h + (x W + b)
    without a gate (the cross-attention branch).  [L, D] -> [L, D]."""
    h = np.asarray(h, dtype=F64)
    z = _lin(np.asarray(x, dtype=F64), wmat, bias)
    return h + z if gate is None else h + gate * z


def cross_q(y2, w, heads):
    """Cross-attention queries y2 Wq2 + bq2: [L, D] -> [L, H, d]."""
    y2 = np.asarray(y2, dtype=F64)
    L, D = y2.shape
    return _lin(y2, w["wq2"], w["bq2"]).reshape(L, heads, D // heads)


def ffn_hidden(y3, w):
    """The FFN's hidden activation GELU_tanh(y3 W1 + b1): [L, D] -> [L, F]."""
    return gelu_tanh(_lin(np.asarray(y3, dtype=F64), w["w1"], w["b1"]))


def qkv_phase(h, mod, w, chunk, grid, heads, trace=None):
    """Self-attention inputs of one task: y = LN(h)(1 + scale1) + shift1;
    q, k, v = y Wqkv + b; RoPE3D on q and k at the chunk's token positions.

    Returns q, k, v, each [L, H, d]; (k, v) is what the chunk leaves in the
    noisy-KV cache at this (block, step).  A dict passed as ``trace`` receives
    the intermediates y1 and q ([L, D])."""
    h = np.asarray(h, dtype=F64)
    L, D = h.shape
    y = adaln(h, mod[0], mod[1])
    q, k, v = qkv_proj(y, w, chunk, grid, heads)
    if trace is not None:
        trace["y1"], trace["q"] = y, q.reshape(L, D)
    return q, k, v


def rest_phase(h, q, K, V, mod, w, ctx_k, ctx_v, rows=None, trace=None):
    """The rest of the block once the window's keys/values are known.

    K, V: [keys, H, d], the window's chunks oldest first then the chunk itself.
      h <- h + gate1 * (Attn(q, K, V) Wo + bo)
      h <- h + CrossAttn(LN(h) Wq2 + bq2, ctx_k, ctx_v) Wo2 + bo2
      h <- h + gate2 * (GELU_tanh((LN(h)(1 + scale2) + shift2) W1 + b1) W2 + b2)
    ``rows`` (optional) restricts the computation to those query rows; every
    step after the attention is row-wise, so the result rows are unchanged.
    A dict passed as ``trace`` receives the intermediates attn, h1, y2, q2,
    xattn, h2, y3 and u (the FFN hidden activation), for those rows."""
    h = np.asarray(h, dtype=F64)
    if rows is not None:
        h = h[rows]
        q = q[rows]
    L, D = h.shape
    heads = q.shape[1]
    a = attention(q, K, V).reshape(L, D)
    h1 = residual(h, a, w["wo"], w["bo"], gate=mod[2])
    y2 = adaln(h1)
    q2 = cross_q(y2, w, heads)
    a2 = attention(q2, ctx_k, ctx_v).reshape(L, D)
    h2 = residual(h1, a2, w["wo2"], w["bo2"])
    y3 = adaln(h2, mod[3], mod[4])
    u = ffn_hidden(y3, w)
    if trace is not None:
        trace.update(attn=a, h1=h1, y2=y2, q2=q2.reshape(L, D), xattn=a2, h2=h2, y3=y3, u=u)
    return residual(h2, u, w["w2"], w["b2"], gate=mod[5])


def block_task(h, e, w, chunk, prior_kv, ctx_kv, grid, heads, rows=None, trace=None):
    """One stage task: block ``w`` at the timestep whose embedding is ``e``.

    prior_kv: list of (K, V) of the window's earlier chunks, oldest first.
    Returns (h_out, (k, v)) where (k, v) is this chunk's cache entry.  A dict
    passed as ``trace`` receives the block's intermediates (qkv_phase and
    rest_phase; y1 and q over all rows, the rest over ``rows``)."""
    mod = modulation(e, w["tmod"])
    q, k, v = qkv_phase(h, mod, w, chunk, grid, heads, trace=trace)
    K = np.concatenate([kv[0] for kv in prior_kv] + [k], axis=0)
    V = np.concatenate([kv[1] for kv in prior_kv] + [v], axis=0)
    h_out = rest_phase(h, q, K, V, mod, w, ctx_kv[0], ctx_kv[1], rows=rows, trace=trace)
    return h_out, (k, v)
