"""Joint placement of streams' virtual ranks onto a GPU pool (binding of
ps_sched_*; the search runs in the native library).

A stream's stages are packed into virtual ranks that take one memory position
of a GPU each; tasks of the same block batch across streams on a GPU; a new
stream is admitted whole, by Best-Fit and Limited Discrepancy Search, only if
it meets its SLO alone, and running streams never move (AREX feed article on
the PhysisServe report, section "三层设计", layer 3; 163.com release, bullet
"虚拟 rank 的动态放置", Fig. 4).
"""
from __future__ import annotations

import ctypes as C
from typing import List, Optional

from . import _lib
from .runtime import check


class Scheduler:
    def __init__(self, n_gpus: int, positions: int, n_blocks: int, n_steps: int, slo_ms: float,
                 batch_fixed_ms: float, batch_task_ms: float, max_discrepancy: int = 2, ranks_per_stream: int = 0):
        self.lib = _lib.load()
        d = _lib.SchedDesc(n_gpus, positions, n_blocks, n_steps, max_discrepancy, ranks_per_stream, slo_ms,
                           batch_fixed_ms, batch_task_ms)
        h = C.c_void_p()
        check(self.lib.ps_sched_create(C.byref(d), C.byref(h)))
        self.handle, self.n_gpus = h, n_gpus

    def split(self) -> int:
        n = C.c_int32()
        check(self.lib.ps_sched_split(self.handle, C.byref(n)))
        return n.value

    def admit(self, stream: int) -> Optional[List[int]]:
        """GPU of each virtual rank if admitted, else None."""
        cap = max(self.split(), 1)
        buf = (C.c_int32 * cap)()
        n = C.c_int32()
        check(self.lib.ps_sched_admit(self.handle, stream, buf, cap, C.byref(n)))
        return list(buf[:n.value]) if n.value else None

    def release(self, stream: int) -> int:
        n = C.c_int32()
        check(self.lib.ps_sched_release(self.handle, stream, C.byref(n)))
        return n.value

    def gpu(self, g: int):
        n, c = C.c_int32(), C.c_double()
        check(self.lib.ps_sched_gpu(self.handle, g, C.byref(n), C.byref(c)))
        return n.value, c.value

    def close(self):
        if self.handle:
            check(self.lib.ps_sched_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def admitted_streams(sched: Scheduler, limit: int = 100000) -> int:
    """Admits streams 0, 1, ... until the first rejection; returns how many."""
    n = 0
    while n < limit and sched.admit(n) is not None:
        n += 1
    return n
