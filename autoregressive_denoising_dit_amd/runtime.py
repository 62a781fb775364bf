"""Python handles over libps.  Torch supplies device memory and streams; every
computation of the stage path runs behind the C ABI in the HIP kernels.
"""
from __future__ import annotations

import ctypes as C
from typing import Dict, Iterable, List, Optional, Sequence

import numpy as np
import torch

from . import _lib
from ._lib import PS_BF16, PS_F32, PS_MAX_WINDOW, Task, check

TORCH_DTYPE = {PS_BF16: torch.bfloat16, PS_F32: torch.float32}


def ps_dtype(name: str) -> int:
    return {"bf16": PS_BF16, "fp32": PS_F32}[name]


def _stream_ptr(stream: Optional[torch.cuda.Stream]) -> C.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> C.c_void_p:
    return C.c_void_p(0 if t is None else t.data_ptr())


def _need(t: torch.Tensor, dtype: torch.dtype, shape: Sequence[int], name: str) -> None:
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: want contiguous {dtype} {tuple(shape)} on the GPU, "
                         f"got {t.dtype} {tuple(t.shape)} (contiguous={t.is_contiguous()}, cuda={t.is_cuda})")


class Pool:
    """The noisy-KV pool (ring slots per (stream, block, step)) plus the cached
    cross-attention keys/values per (stream, block)."""

    def __init__(self, n_streams: int, n_blocks: int, n_steps: int, n_slots: int, grid, n_heads: int,
                 head_dim: int, max_ctx: int, dtype: int, check_slots: bool = False):
        self.lib = _lib.load()
        self.grid = tuple(grid)
        self.tokens = grid[0] * grid[1] * grid[2]
        self.n_heads, self.head_dim, self.dtype = n_heads, head_dim, dtype
        self.hidden = n_heads * head_dim
        self.n_slots, self.max_ctx = n_slots, max_ctx
        d = _lib.PoolDesc(n_streams, n_blocks, n_steps, n_slots, grid[0], grid[1], grid[2],
                          n_heads, head_dim, max_ctx, dtype, 1 if check_slots else 0)
        h = C.c_void_p()
        check(self.lib.ps_kv_pool_create(C.byref(d), C.byref(h)))
        self.handle = h

    def close(self):
        if self.handle:
            check(self.lib.ps_kv_pool_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _kv_shape(self, n=None):
        return (self.tokens if n is None else n, self.n_heads, self.head_dim)

    def load(self, stream: int, block: int, step: int, slot: int, chunk: int, k: torch.Tensor,
             v: torch.Tensor, cuda_stream=None):
        td = TORCH_DTYPE[self.dtype]
        _need(k, td, self._kv_shape(), "k")
        _need(v, td, self._kv_shape(), "v")
        check(self.lib.ps_kv_pool_load(self.handle, stream, block, step, slot, chunk, _ptr(k), _ptr(v),
                                       _stream_ptr(cuda_stream)))

    def fetch(self, stream: int, block: int, step: int, slot: int, cuda_stream=None):
        td = TORCH_DTYPE[self.dtype]
        k = torch.empty(self._kv_shape(), dtype=td, device="cuda")
        v = torch.empty_like(k)
        check(self.lib.ps_kv_pool_fetch(self.handle, stream, block, step, slot, _ptr(k), _ptr(v),
                                        _stream_ptr(cuda_stream)))
        return k, v

    def context_fetch(self, stream: int, block: int, n_ctx: int, cuda_stream=None):
        td = TORCH_DTYPE[self.dtype]
        k = torch.empty(self._kv_shape(n_ctx), dtype=td, device="cuda")
        v = torch.empty_like(k)
        check(self.lib.ps_context_fetch(self.handle, stream, block, _ptr(k), _ptr(v),
                                        _stream_ptr(cuda_stream)))
        return k, v

    def context_load(self, stream: int, block: int, k: torch.Tensor, v: torch.Tensor, cuda_stream=None):
        """Stores given cross-attention keys/values [n_ctx, H, d] of (stream, block)."""
        td = TORCH_DTYPE[self.dtype]
        n = k.shape[0]
        _need(k, td, self._kv_shape(n), "k")
        _need(v, td, self._kv_shape(n), "v")
        check(self.lib.ps_context_load(self.handle, stream, block, _ptr(k), _ptr(v), n, _stream_ptr(cuda_stream)))

    def release_stream(self, cuda_stream) -> None:
        """Waits for the stream and frees the workspace the pool keeps for it."""
        check(self.lib.ps_kv_pool_release_stream(self.handle, _stream_ptr(cuda_stream)))

    def context_set(self, block: "Block", stream: int, ctx: torch.Tensor, cuda_stream=None):
        _need(ctx, TORCH_DTYPE[self.dtype], (ctx.shape[0], self.hidden), "ctx")
        check(self.lib.ps_context_set(self.handle, block.handle, stream, _ptr(ctx), ctx.shape[0],
                                      _stream_ptr(cuda_stream)))


_BLOCK_MATS = ("wqkv", "wo", "wq2", "wkv2", "wo2", "w1", "w2")
_BLOCK_VECS = ("bqkv", "bo", "bq2", "bkv2", "bo2", "b1", "b2", "tmod")


class Block:
    """One DiT block's weights on the device: matrices [out, in] in the compute
    dtype, biases and the modulation table fp32.  The tensors are kept alive
    for as long as the handle."""

    def __init__(self, tensors: Dict[str, torch.Tensor], hidden: int, n_heads: int, head_dim: int,
                 ffn: int, block_index: int, dtype: int):
        self.lib = _lib.load()
        D, F = hidden, ffn
        td = TORCH_DTYPE[dtype]
        shapes = {"wqkv": (3 * D, D), "wo": (D, D), "wq2": (D, D), "wkv2": (2 * D, D), "wo2": (D, D),
                  "w1": (F, D), "w2": (D, F), "bqkv": (3 * D,), "bo": (D,), "bq2": (D,), "bkv2": (2 * D,),
                  "bo2": (D,), "b1": (F,), "b2": (D,), "tmod": (6, D)}
        for k in _BLOCK_MATS:
            _need(tensors[k], td, shapes[k], k)
        for k in _BLOCK_VECS:
            _need(tensors[k], torch.float32, shapes[k], k)
        self.tensors = tensors
        self.hidden, self.ffn, self.block_index, self.dtype = hidden, ffn, block_index, dtype
        d = _lib.BlockDesc(hidden, n_heads, head_dim, ffn, block_index, dtype,
                           *[tensors[k].data_ptr() for k in _BLOCK_MATS],
                           *[tensors[k].data_ptr() for k in _BLOCK_VECS])
        h = C.c_void_p()
        check(self.lib.ps_block_create(C.byref(d), C.byref(h)))
        self.handle = h

    @classmethod
    def from_numpy(cls, w: Dict[str, np.ndarray], hidden: int, n_heads: int, head_dim: int, ffn: int,
                   block_index: int, dtype: int, device="cuda"):
        """Uploads weights given as [in, out] arrays (y = x @ W + b)."""
        td = TORCH_DTYPE[dtype]
        t = {}
        for k in _BLOCK_MATS:
            t[k] = torch.from_numpy(np.ascontiguousarray(np.asarray(w[k], np.float32).T)).to(device, td).contiguous()
        for k in _BLOCK_VECS:
            t[k] = torch.from_numpy(np.ascontiguousarray(np.asarray(w[k], np.float32))).to(device)
        return cls(t, hidden, n_heads, head_dim, ffn, block_index, dtype)

    def close(self):
        if self.handle:
            check(self.lib.ps_block_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class TimeEmbed:
    """Shared timestep MLP + D -> 6D projection (fp32, [out, in]) with a cache of e(t)."""

    def __init__(self, tensors: Dict[str, torch.Tensor], hidden: int, capacity: int = 16):
        self.lib = _lib.load()
        D = hidden
        shapes = {"wt1": (D, _lib.PS_FREQ_DIM), "bt1": (D,), "wt2": (D, D), "bt2": (D,), "wp": (6 * D, D),
                  "bp": (6 * D,)}
        for k, s in shapes.items():
            _need(tensors[k], torch.float32, s, k)
        self.tensors, self.hidden = tensors, hidden
        d = _lib.TimeDesc(hidden, capacity, *[tensors[k].data_ptr() for k in ("wt1", "bt1", "wt2", "bt2", "wp", "bp")])
        h = C.c_void_p()
        check(self.lib.ps_time_embed_create(C.byref(d), C.byref(h)))
        self.handle = h

    @classmethod
    def from_numpy(cls, w: Dict[str, np.ndarray], hidden: int, capacity: int = 16, device="cuda"):
        t = {}
        for k in ("wt1", "wt2", "wp"):
            t[k] = torch.from_numpy(np.ascontiguousarray(np.asarray(w[k], np.float32).T)).to(device)
        for k in ("bt1", "bt2", "bp"):
            t[k] = torch.from_numpy(np.ascontiguousarray(np.asarray(w[k], np.float32))).to(device)
        return cls(t, hidden, capacity)

    def get(self, t: float, cuda_stream=None) -> torch.Tensor:
        e = torch.empty((6, self.hidden), dtype=torch.float32, device="cuda")
        check(self.lib.ps_time_embed_get(self.handle, C.c_float(t), _ptr(e), _stream_ptr(cuda_stream)))
        return e

    def close(self):
        if self.handle:
            check(self.lib.ps_time_embed_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Head:
    """Patch embedding and output head on the device: w_embed [D, P] and w_head
    [P, D] in the compute dtype ([out, in]); b_embed [D], b_head [P], t_head
    [2, D] fp32.  The tensors are kept alive for as long as the handle."""

    def __init__(self, tensors: Dict[str, torch.Tensor], hidden: int, latent_dim: int, dtype: int):
        self.lib = _lib.load()
        D, P = hidden, latent_dim
        td = TORCH_DTYPE[dtype]
        _need(tensors["w_embed"], td, (D, P), "w_embed")
        _need(tensors["w_head"], td, (P, D), "w_head")
        _need(tensors["b_embed"], torch.float32, (D,), "b_embed")
        _need(tensors["b_head"], torch.float32, (P,), "b_head")
        _need(tensors["t_head"], torch.float32, (2, D), "t_head")
        self.tensors, self.hidden, self.latent_dim, self.dtype = tensors, D, P, dtype
        d = _lib.HeadDesc(D, P, dtype, *[tensors[k].data_ptr()
                                         for k in ("w_embed", "w_head", "b_embed", "b_head", "t_head")])
        h = C.c_void_p()
        check(self.lib.ps_head_create(C.byref(d), C.byref(h)))
        self.handle = h

    @classmethod
    def from_numpy(cls, w: Dict[str, np.ndarray], hidden: int, latent_dim: int, dtype: int, device="cuda"):
        """Uploads weights given as [in, out] arrays (y = x @ W + b)."""
        td = TORCH_DTYPE[dtype]
        t = {k: torch.from_numpy(np.ascontiguousarray(np.asarray(w[k], np.float32).T)).to(device, td).contiguous()
             for k in ("w_embed", "w_head")}
        for k in ("b_embed", "b_head", "t_head"):
            t[k] = torch.from_numpy(np.ascontiguousarray(np.asarray(w[k], np.float32))).to(device)
        return cls(t, hidden, latent_dim, dtype)

    def close(self):
        if self.handle:
            check(self.lib.ps_head_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def patch_embed(head: Head, x: torch.Tensor, h: torch.Tensor, cuda_stream=None) -> None:
    """h = x W_embed^T + b_embed for latent patches x [rows, P] (fp32) -> h [rows, D] (fp32)."""
    rows = x.shape[0]
    _need(x, torch.float32, (rows, head.latent_dim), "x")
    _need(h, torch.float32, (rows, head.hidden), "h")
    check(head.lib.ps_patch_embed(head.handle, _ptr(x), _ptr(h), rows, _stream_ptr(cuda_stream)))


def output_head(head: Head, te: TimeEmbed, timesteps: Sequence[float], tokens: int, h: torch.Tensor,
                v: torch.Tensor, cuda_stream=None) -> None:
    """v = head(h) per task (tokens rows each, timestep timesteps[i]): h [n * tokens, D] -> v [n * tokens, P]."""
    n = len(timesteps)
    _need(h, torch.float32, (n * tokens, head.hidden), "h")
    _need(v, torch.float32, (n * tokens, head.latent_dim), "v")
    arr = (C.c_float * n)(*[float(t) for t in timesteps])
    check(head.lib.ps_output_head(head.handle, te.handle, arr, n, tokens, _ptr(h), _ptr(v), _stream_ptr(cuda_stream)))


def make_task(stream: int, chunk: int, step: int, timestep: float, write_slot: int,
              read_slots: Iterable[int]) -> Task:
    rs = list(read_slots)
    if len(rs) > PS_MAX_WINDOW:
        raise ValueError("too many read slots")
    t = Task()
    t.stream, t.chunk, t.step, t.timestep = stream, chunk, step, float(timestep)
    t.write_slot, t.n_read = write_slot, len(rs)
    for i, s in enumerate(rs):
        t.read_slots[i] = s
    return t


def stage_batch(pool: Pool, block: Block, te: TimeEmbed, tasks: List[Task], h_in: torch.Tensor,
                h_out: torch.Tensor, cuda_stream=None) -> None:
    n = len(tasks)
    _need(h_in, torch.float32, (n * pool.tokens, pool.hidden), "h_in")
    _need(h_out, torch.float32, (n * pool.tokens, pool.hidden), "h_out")
    arr = (Task * max(n, 1))(*tasks)
    check(pool.lib.ps_stage_batch(pool.handle, block.handle, te.handle, arr, n, _ptr(h_in), _ptr(h_out),
                                  _stream_ptr(cuda_stream)))


def stage_batch_rows(pool: Pool, block: Block, te: TimeEmbed, tasks: List[Task], h_in: Sequence[torch.Tensor],
                     h_out: Sequence[torch.Tensor], cuda_stream=None) -> None:
    """stage_batch on tasks whose rows live in separate tensors: h_in[i],
    h_out[i] fp32 [L, D] (ps_stage_batch_rows)."""
    n = len(tasks)
    if len(h_in) != n or len(h_out) != n:
        raise ValueError("one input and one output row tensor per task")
    for i in range(n):
        _need(h_in[i], torch.float32, (pool.tokens, pool.hidden), f"h_in[{i}]")
        _need(h_out[i], torch.float32, (pool.tokens, pool.hidden), f"h_out[{i}]")
    arr = (Task * max(n, 1))(*tasks)
    pin = (C.c_void_p * n)(*[t.data_ptr() for t in h_in])
    pout = (C.c_void_p * n)(*[t.data_ptr() for t in h_out])
    check(pool.lib.ps_stage_batch_rows(pool.handle, block.handle, te.handle, arr, n, pin, pout,
                                       _stream_ptr(cuda_stream)))


def stage_batch_static(pool: Pool, block: Block, te: TimeEmbed, tasks: List[Task], h_in: torch.Tensor,
                       h_out: torch.Tensor, cuda_stream=None) -> None:
    """stage_batch without device allocation (ps_stage_batch_static): the
    workspace is the library's fixed per-device array."""
    n = len(tasks)
    _need(h_in, torch.float32, (n * pool.tokens, pool.hidden), "h_in")
    _need(h_out, torch.float32, (n * pool.tokens, pool.hidden), "h_out")
    arr = (Task * max(n, 1))(*tasks)
    check(pool.lib.ps_stage_batch_static(pool.handle, block.handle, te.handle, arr, n, _ptr(h_in), _ptr(h_out),
                                         _stream_ptr(cuda_stream)))


def stage_batch_probe(pool: Pool, block: Block, te: TimeEmbed, tasks: List[Task], h_in: torch.Tensor,
                      h_out: torch.Tensor, probe: Dict[str, torch.Tensor], cuda_stream=None) -> None:
    """stage_batch that also copies the intermediates named in `probe`
    (keys from _lib.PROBE_FIELDS, each a dense device tensor: [n*L, F] for
    "u", [n*L, D] otherwise; fp32 for h1 / h2, the compute dtype otherwise)."""
    n = len(tasks)
    _need(h_in, torch.float32, (n * pool.tokens, pool.hidden), "h_in")
    _need(h_out, torch.float32, (n * pool.tokens, pool.hidden), "h_out")
    pr = _lib.StageProbe()
    for name, t in probe.items():
        if name not in _lib.PROBE_FIELDS:
            raise ValueError(f"unknown probe member {name!r}")
        dt = torch.float32 if name in _lib.PROBE_FP32 else TORCH_DTYPE[block.dtype]
        cols = block.ffn if name == "u" else pool.hidden
        _need(t, dt, (n * pool.tokens, cols), name)
        setattr(pr, name, t.data_ptr())
    arr = (Task * max(n, 1))(*tasks)
    check(pool.lib.ps_stage_batch_probe(pool.handle, block.handle, te.handle, arr, n, _ptr(h_in), _ptr(h_out),
                                        C.byref(pr), _stream_ptr(cuda_stream)))


def stage_kernel(pool: Pool, block: Block, te: TimeEmbed, tasks: List[Task], kernel: str, x: torch.Tensor,
                 out: torch.Tensor, h_in: Optional[torch.Tensor] = None, cuda_stream=None) -> None:
    """One kernel of the stage (_lib.KERNELS) on the given input x; see
    ps_stage_kernel for each kernel's input, residual input and output."""
    n = len(tasks)
    M, D, F = n * pool.tokens, pool.hidden, block.ffn
    td = TORCH_DTYPE[block.dtype]
    k = _lib.KERNELS.index(kernel)
    fp_in = kernel in ("ln1", "ln2", "ln3")
    fp_out = kernel in ("o_proj", "xo_proj", "ffn2")
    _need(x, torch.float32 if fp_in else td, (M, F if kernel == "ffn2" else D), "x")
    _need(out, torch.float32 if fp_out else td, (M, F if kernel == "ffn1" else D), "out")
    if fp_out:
        if h_in is None:
            raise ValueError(f"{kernel} needs h_in")
        _need(h_in, torch.float32, (M, D), "h_in")
    arr = (Task * max(n, 1))(*tasks)
    check(pool.lib.ps_stage_kernel(pool.handle, block.handle, te.handle, arr, n, k, _ptr(x), _ptr(h_in), _ptr(out),
                                   _stream_ptr(cuda_stream)))


def timesteps(n_steps: int, shift: float = 1.0) -> List[float]:
    """t_0 .. t_{S-1} of an S-step schedule under the flow-matching time shift
    (ps_timesteps; the list leaves out t_S = 0)."""
    out = (C.c_float * (n_steps + 1))()
    check(_lib.load().ps_timesteps(n_steps, C.c_float(shift), out))
    return [float(out[i]) for i in range(n_steps)]


def euler_update_steps(x: torch.Tensor, v: torch.Tensor, ts: Sequence[float], steps: Sequence[int], tokens: int,
                       hidden: int, cuda_stream=None) -> None:
    """Euler step of each task with dt taken from the schedule ts (t_S = 0) at
    the task's step (ps_euler_update_steps)."""
    n = len(steps)
    _need(x, torch.float32, (n * tokens, hidden), "x")
    if v.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("v must be fp32 or bf16")
    _need(v, v.dtype, (n * tokens, hidden), "v")
    vdt = PS_F32 if v.dtype == torch.float32 else PS_BF16
    tarr = (C.c_float * len(ts))(*[float(t) for t in ts])
    sarr = (C.c_int32 * n)(*[int(s) for s in steps])
    check(_lib.load().ps_euler_update_steps(_ptr(x), _ptr(v), tarr, len(ts), sarr, n, tokens, hidden, vdt,
                                            _stream_ptr(cuda_stream)))


def euler_update(x: torch.Tensor, v: torch.Tensor, dt: Sequence[float], tokens: int, hidden: int,
                 cuda_stream=None) -> None:
    n = len(dt)
    _need(x, torch.float32, (n * tokens, hidden), "x")
    if v.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("v must be fp32 or bf16")
    _need(v, v.dtype, (n * tokens, hidden), "v")
    vdt = PS_F32 if v.dtype == torch.float32 else PS_BF16
    arr = (C.c_float * n)(*[float(x_) for x_ in dt])
    check(_lib.load().ps_euler_update(_ptr(x), _ptr(v), arr, n, tokens, hidden, vdt, _stream_ptr(cuda_stream)))
