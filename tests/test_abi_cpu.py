"""The C-ABI library without a GPU: it loads, exports every call include/ps.h
declares, its structs match the ctypes mirror, and argument validation fails
before any device work.  Also the host-side schedule logic."""
import ctypes as C
import os
import re
import shutil
import subprocess

import pytest

from autoregressive_denoising_dit_amd import _lib
from autoregressive_denoising_dit_amd.schedule import n_ticks, tick_tasks

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

needs_lib = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libps.so not built")


def header_functions():
    txt = "".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"^\s*(?:ps_status|const char\*|int32_t)\s+(ps_\w+)\s*\(", txt, re.M)))


def test_header_lists_the_binding_exports():
    assert header_functions() == sorted(_lib.EXPORTS)


@needs_lib
def test_library_exports_every_declared_symbol():
    assert sorted(_lib.exported_symbols()) == header_functions()


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc missing")
def test_struct_layout_matches_ctypes(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(r'''
#include <stdio.h>
#include <stddef.h>
#include "ps.h"
#include "ps_sched.h"
int main(void) {
  printf("%zu %zu %zu %zu\n", sizeof(ps_pool_desc), sizeof(ps_block_desc), sizeof(ps_time_desc), sizeof(ps_task));
  printf("%zu %zu %zu %zu\n", offsetof(ps_block_desc, wqkv), offsetof(ps_block_desc, tmod),
         offsetof(ps_time_desc, wt1), offsetof(ps_task, read_slots));
  printf("%zu %zu %zu %zu\n", sizeof(ps_head_desc), offsetof(ps_head_desc, w_embed), sizeof(ps_sched_desc),
         offsetof(ps_sched_desc, slo_ms));
  printf("%zu %zu %zu\n", sizeof(ps_stage_probe), offsetof(ps_stage_probe, h1), offsetof(ps_stage_probe, u));
  return 0;
}
''')
    exe = tmp_path / "layout"
    r = subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                        "-I", "/opt/rocm/include", str(src), "-o", str(exe)], capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("cannot compile against hip_runtime_api.h: " + r.stderr[:200])
    out = subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()
    got = [int(x) for x in out]
    want = [C.sizeof(_lib.PoolDesc), C.sizeof(_lib.BlockDesc), C.sizeof(_lib.TimeDesc), C.sizeof(_lib.Task),
            _lib.BlockDesc.wqkv.offset, _lib.BlockDesc.tmod.offset, _lib.TimeDesc.wt1.offset,
            _lib.Task.read_slots.offset, C.sizeof(_lib.HeadDesc), _lib.HeadDesc.w_embed.offset,
            C.sizeof(_lib.SchedDesc), _lib.SchedDesc.slo_ms.offset,
            C.sizeof(_lib.StageProbe), _lib.StageProbe.h1.offset, _lib.StageProbe.u.offset]
    assert got == want


@needs_lib
def test_validation_fails_before_device_work():
    lib = _lib.load()
    h = C.c_void_p()
    bad_pools = [
        _lib.PoolDesc(0, 1, 1, 1, 1, 8, 8, 2, 64, 16, 0, 0),      # no streams
        _lib.PoolDesc(1, 1, 1, 1, 1, 3, 5, 2, 64, 16, 0, 0),      # 15 tokens: not a multiple of 8
        _lib.PoolDesc(1, 1, 1, 1, 1, 4, 8, 2, 64, 16, 0, 0),      # 32 tokens: below one key tile
        _lib.PoolDesc(1, 1, 1, 1, 1, 8, 8, 2, 96, 16, 0, 0),      # head_dim 96
        _lib.PoolDesc(1, 1, 1, 1, 1, 8, 8, 2, 64, 12, 0, 0),      # max_ctx not a multiple of 8
        _lib.PoolDesc(1, 1, 1, 1, 1, 8, 8, 2, 64, 16, 7, 0),      # dtype
    ]
    for d in bad_pools:
        assert lib.ps_kv_pool_create(C.byref(d), C.byref(h)) == _lib.PS_ERR_INVALID_ARG
        assert lib.ps_last_error()
    bd = _lib.BlockDesc(128, 2, 64, 512, 0, 0)                   # null weights
    assert lib.ps_block_create(C.byref(bd), C.byref(h)) == _lib.PS_ERR_INVALID_ARG
    bd = _lib.BlockDesc(120, 2, 64, 512, 0, 0, *([16] * 15))     # hidden != heads * head_dim
    assert lib.ps_block_create(C.byref(bd), C.byref(h)) == _lib.PS_ERR_INVALID_ARG
    bd = _lib.BlockDesc(128, 2, 64, 500, 0, 1, *([16] * 15))     # ffn not a multiple of 64 (bf16)
    assert lib.ps_block_create(C.byref(bd), C.byref(h)) == _lib.PS_ERR_INVALID_ARG
    td = _lib.TimeDesc(128, 0, *([16] * 6))                     # zero capacity
    assert lib.ps_time_embed_create(C.byref(td), C.byref(h)) == _lib.PS_ERR_INVALID_ARG
    assert lib.ps_stage_batch(None, None, None, None, 1, None, None, None) == _lib.PS_ERR_INVALID_ARG
    assert lib.ps_stage_batch_probe(None, None, None, None, 1, None, None, None, None) == _lib.PS_ERR_INVALID_ARG
    assert b"probe" in lib.ps_last_error()
    pr = _lib.StageProbe()
    assert lib.ps_stage_batch_probe(None, None, None, None, 1, None, None, C.byref(pr), None) == _lib.PS_ERR_INVALID_ARG
    dt = (C.c_float * 1)(0.5)
    assert lib.ps_euler_update(None, None, dt, 1, 64, 128, 0, None) == _lib.PS_ERR_INVALID_ARG
    assert lib.ps_euler_update(C.c_void_p(16), C.c_void_p(16), dt, 0, 64, 128, 0, None) == _lib.PS_ERR_INVALID_ARG
    dt_nan = (C.c_float * 1)(float("nan"))
    assert lib.ps_euler_update(C.c_void_p(16), C.c_void_p(16), dt_nan, 1, 64, 128, 0, None) == _lib.PS_ERR_INVALID_ARG
    assert b"finite" in lib.ps_last_error()


# ------------------------------------------------------------ host schedule
@pytest.mark.parametrize("k,n_streams", [(1, 1), (2, 1), (1, 3), (3, 2)])
def test_tick_tasks_cover_schedule(k, n_streams):
    S, N = 4, 11
    seen = []
    for tau in range(n_ticks(N, S, k)):
        tl = tick_tasks(tau, N, S, k, n_streams)
        seen += tl
        # chunk-major, stream-minor, chunks contiguous: the tick's rows are one slice
        assert tl == sorted(tl, key=lambda t: (t[1], t[0]))
        cs = sorted({c for (_, c, _) in tl})
        assert cs == list(range(cs[0], cs[-1] + 1)) if cs else True
        assert len(tl) == len(cs) * n_streams
        for (sg, c, s) in tl:
            assert c == k * (tau - s) + (c % k)
    assert sorted(seen) == sorted((sg, c, s) for sg in range(n_streams) for c in range(N) for s in range(S))


def test_tick_tasks_match_oracle_definition():
    import oracle
    for k in (1, 2):
        ref = oracle.staggered_ticks(9, 4, k, 2)
        for tau, tasks in enumerate(ref):
            assert sorted(tick_tasks(tau, 9, 4, k, 2)) == sorted(tasks)


@pytest.mark.parametrize("S,shift", [(4, 1.0), (4, 3.0), (7, 5.0), (1, 2.0)])
def test_shifted_timesteps_match_the_oracle(S, shift):
    import oracle
    from autoregressive_denoising_dit_amd.schedule import shifted_timesteps
    got, ref = shifted_timesteps(S, shift), oracle.shifted_timesteps(S, shift)
    assert len(got) == S
    # the library returns fp32 timesteps (a task's timestep is fp32): the
    # oracle's value rounded to fp32, give or take one ulp at a rounding tie
    for a, b in zip(got, ref):
        assert a == pytest.approx(b, rel=2.0 ** -23, abs=0)


def test_new_entry_points_reject_bad_arguments():
    """Host-side validation of the calls that need no GPU to reject."""
    lib = _lib.load()
    out = (C.c_float * 5)()
    assert lib.ps_timesteps(0, C.c_float(1.0), out) == _lib.PS_ERR_INVALID_ARG
    assert lib.ps_timesteps(4, C.c_float(0.0), out) == _lib.PS_ERR_INVALID_ARG
    assert lib.ps_timesteps(4, C.c_float(float("nan")), out) == _lib.PS_ERR_INVALID_ARG
    assert lib.ps_timesteps(4, C.c_float(1.0), None) == _lib.PS_ERR_INVALID_ARG
    assert lib.ps_timesteps(4, C.c_float(1.0), out) == _lib.PS_OK
    assert list(out) == [1.0, 0.75, 0.5, 0.25, 0.0]
    ts = (C.c_float * 4)(1.0, 0.75, 0.5, 0.25)
    steps = (C.c_int32 * 1)(4)                                   # step out of range
    assert lib.ps_euler_update_steps(C.c_void_p(16), C.c_void_p(16), ts, 4, steps, 1, 64, 128, 0,
                                     None) == _lib.PS_ERR_INVALID_ARG
    assert b"out of range" in lib.ps_last_error()
    assert lib.ps_euler_update_steps(C.c_void_p(16), C.c_void_p(16), None, 4, steps, 1, 64, 128, 0,
                                     None) == _lib.PS_ERR_INVALID_ARG
    assert lib.ps_stage_kernel(None, None, None, None, 1, 99, None, None, None, None) == _lib.PS_ERR_INVALID_ARG
    assert b"unknown kernel" in lib.ps_last_error()
    assert lib.ps_stage_kernel(None, None, None, None, 1, 3, None, None, None, None) == _lib.PS_ERR_INVALID_ARG
    assert lib.ps_context_load(None, 0, 0, None, None, 8, None) == _lib.PS_ERR_INVALID_ARG
    assert lib.ps_kv_pool_release_stream(None, None) == _lib.PS_ERR_INVALID_ARG
