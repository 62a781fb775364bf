"""ctypes binding of libps (include/ps.h): argument marshalling only.

Every step of the stage path runs in the HIP kernels behind the C ABI; this
module only mirrors the header's structs and turns a non-zero ps_status into
an exception.  It fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libps.so")

PS_OK = 0
PS_ERR_INVALID_ARG = -1
PS_ERR_OUT_OF_MEMORY = -2
PS_ERR_HIP = -3
PS_ERR_SLOT_CONFLICT = -4
PS_ERR_UNSUPPORTED = -5
STATUS_NAMES = {0: "PS_OK", -1: "PS_ERR_INVALID_ARG", -2: "PS_ERR_OUT_OF_MEMORY", -3: "PS_ERR_HIP",
                -4: "PS_ERR_SLOT_CONFLICT", -5: "PS_ERR_UNSUPPORTED"}

PS_F32 = 0
PS_BF16 = 1
# ps_stage_kernel's kernels, in stage order
KERNELS = ("ln1", "qkv", "attn_self", "o_proj", "ln2", "xq_proj", "attn_cross", "xo_proj", "ln3", "ffn1", "ffn2")
PS_MAX_WINDOW = 8
PS_MAX_TASKS = 32
PS_FREQ_DIM = 256
PS_STATIC_SCRATCH_BYTES = 128 << 20

EXPORTS = (
    "ps_kv_pool_create", "ps_kv_pool_destroy", "ps_kv_pool_load", "ps_kv_pool_fetch",
    "ps_context_fetch", "ps_block_create", "ps_block_destroy", "ps_time_embed_create",
    "ps_time_embed_destroy", "ps_time_embed_get", "ps_context_set", "ps_stage_batch", "ps_stage_batch_probe",
    "ps_euler_update", "ps_last_error", "ps_trace_enable", "ps_trace_collect", "ps_trace_count",
    "ps_trace_entry", "ps_head_create", "ps_head_destroy", "ps_patch_embed", "ps_output_head",
    "ps_sched_create", "ps_sched_destroy", "ps_sched_split", "ps_sched_admit", "ps_sched_release",
    "ps_sched_gpu", "ps_kv_pool_release_stream", "ps_context_load", "ps_stage_kernel", "ps_timesteps",
    "ps_euler_update_steps", "ps_stage_batch_static", "ps_stage_batch_rows",
)


class PsError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class PoolDesc(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "n_streams", "n_blocks", "n_steps", "n_slots", "frames", "rows", "cols",
        "n_heads", "head_dim", "max_ctx", "dtype", "check_slots")]


class BlockDesc(C.Structure):
    _fields_ = ([(n, C.c_int32) for n in ("hidden", "n_heads", "head_dim", "ffn", "block_index", "dtype")]
                + [(n, C.c_void_p) for n in ("wqkv", "wo", "wq2", "wkv2", "wo2", "w1", "w2")]
                + [(n, C.c_void_p) for n in ("bqkv", "bo", "bq2", "bkv2", "bo2", "b1", "b2", "tmod")])


class TimeDesc(C.Structure):
    _fields_ = ([("hidden", C.c_int32), ("capacity", C.c_int32)]
                + [(n, C.c_void_p) for n in ("wt1", "bt1", "wt2", "bt2", "wp", "bp")])


class HeadDesc(C.Structure):
    _fields_ = ([("hidden", C.c_int32), ("latent_dim", C.c_int32), ("dtype", C.c_int32)]
                + [(n, C.c_void_p) for n in ("w_embed", "w_head", "b_embed", "b_head", "t_head")])


class SchedDesc(C.Structure):
    _fields_ = [("n_gpus", C.c_int32), ("positions", C.c_int32), ("n_blocks", C.c_int32), ("n_steps", C.c_int32),
                ("max_discrepancy", C.c_int32), ("ranks_per_stream", C.c_int32), ("slo_ms", C.c_double),
                ("batch_fixed_ms", C.c_double), ("batch_task_ms", C.c_double)]


PROBE_FIELDS = ("y1", "q", "attn", "h1", "y2", "q2", "xattn", "h2", "y3", "u")
PROBE_FP32 = ("h1", "h2")   # the others are in the compute dtype


class StageProbe(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in PROBE_FIELDS]


class Task(C.Structure):
    _fields_ = [("stream", C.c_int32), ("chunk", C.c_int32), ("step", C.c_int32),
                ("timestep", C.c_float), ("write_slot", C.c_int32), ("n_read", C.c_int32),
                ("read_slots", C.c_int32 * PS_MAX_WINDOW)]


_lib = None


def load(path: str = LIB_PATH) -> C.CDLL:
    """Loads libps.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build the HIP library first "
            "(python -m autoregressive_denoising_dit_amd.build)")
    lib = C.CDLL(path)
    vp, i32, f32 = C.c_void_p, C.c_int32, C.c_float
    sig = {
        "ps_kv_pool_create": [C.POINTER(PoolDesc), C.POINTER(vp)],
        "ps_kv_pool_destroy": [vp],
        "ps_kv_pool_load": [vp, i32, i32, i32, i32, i32, vp, vp, vp],
        "ps_kv_pool_fetch": [vp, i32, i32, i32, i32, vp, vp, vp],
        "ps_context_fetch": [vp, i32, i32, vp, vp, vp],
        "ps_block_create": [C.POINTER(BlockDesc), C.POINTER(vp)],
        "ps_block_destroy": [vp],
        "ps_time_embed_create": [C.POINTER(TimeDesc), C.POINTER(vp)],
        "ps_time_embed_destroy": [vp],
        "ps_time_embed_get": [vp, f32, vp, vp],
        "ps_context_set": [vp, vp, i32, vp, i32, vp],
        "ps_stage_batch": [vp, vp, vp, C.POINTER(Task), i32, vp, vp, vp],
        "ps_stage_batch_probe": [vp, vp, vp, C.POINTER(Task), i32, vp, vp, C.POINTER(StageProbe), vp],
        "ps_euler_update": [vp, vp, C.POINTER(C.c_float), i32, i32, i32, i32, vp],
        "ps_head_create": [C.POINTER(HeadDesc), C.POINTER(vp)],
        "ps_head_destroy": [vp],
        "ps_patch_embed": [vp, vp, vp, i32, vp],
        "ps_output_head": [vp, vp, C.POINTER(C.c_float), i32, i32, vp, vp, vp],
        "ps_sched_create": [C.POINTER(SchedDesc), C.POINTER(vp)],
        "ps_sched_destroy": [vp],
        "ps_sched_split": [vp, C.POINTER(i32)],
        "ps_sched_admit": [vp, C.c_int64, C.POINTER(i32), i32, C.POINTER(i32)],
        "ps_sched_release": [vp, C.c_int64, C.POINTER(i32)],
        "ps_sched_gpu": [vp, i32, C.POINTER(i32), C.POINTER(C.c_double)],
        "ps_kv_pool_release_stream": [vp, vp],
        "ps_context_load": [vp, i32, i32, vp, vp, i32, vp],
        "ps_stage_kernel": [vp, vp, vp, C.POINTER(Task), i32, i32, vp, vp, vp, vp],
        "ps_timesteps": [i32, f32, C.POINTER(C.c_float)],
        "ps_euler_update_steps": [vp, vp, C.POINTER(C.c_float), i32, C.POINTER(i32), i32, i32, i32, i32, vp],
        "ps_stage_batch_static": [vp, vp, vp, C.POINTER(Task), i32, vp, vp, vp],
        "ps_stage_batch_rows": [vp, vp, vp, C.POINTER(Task), i32, C.POINTER(vp), C.POINTER(vp), vp],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = i32
    lib.ps_last_error.argtypes = []
    lib.ps_last_error.restype = C.c_char_p
    lib.ps_trace_enable.argtypes = [i32]
    lib.ps_trace_enable.restype = i32
    lib.ps_trace_collect.argtypes = []
    lib.ps_trace_collect.restype = i32
    lib.ps_trace_count.argtypes = []
    lib.ps_trace_count.restype = i32
    lib.ps_trace_entry.argtypes = [i32, C.POINTER(C.c_char_p), C.POINTER(C.c_int64), C.POINTER(C.c_double)]
    lib.ps_trace_entry.restype = i32
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != PS_OK:
        msg = load().ps_last_error().decode(errors="replace")
        raise PsError(status, msg)


def trace_enable(on: bool) -> None:
    check(load().ps_trace_enable(1 if on else 0))


def trace_read() -> dict:
    """{kernel name: (launches, total ms)} accumulated since trace_enable(True)."""
    lib = load()
    check(lib.ps_trace_collect())
    out = {}
    for i in range(lib.ps_trace_count()):
        name, n, ms = C.c_char_p(), C.c_int64(), C.c_double()
        check(lib.ps_trace_entry(i, C.byref(name), C.byref(n), C.byref(ms)))
        out[name.value.decode()] = (n.value, ms.value)
    return out


def exported_symbols(path: str = LIB_PATH):
    """Names from EXPORTS that the shared object defines (no GPU needed)."""
    lib = C.CDLL(path)
    return [n for n in EXPORTS if hasattr(lib, n)]
