"""MI355X-native stage-task path of an autoregressive-denoising DiT server.

The compute runs in hand-written gfx950 HIP kernels behind the C ABI of
``libps.so`` (declared in ``include/ps.h``); this package holds the ctypes
binding (``_lib``), thin torch-facing handles (``runtime``), the staggered
chunk x step driver (``schedule``) and the build script (``build``).
"""
from . import _lib  # noqa: F401

__all__ = ["_lib", "runtime", "schedule", "build"]
