"""Workload shapes and seeded synthetic inputs shared by the oracle and the GPU path.

Holds sizes and random draws only -- none of the method's arithmetic."""
from . import configs, inputs  # noqa: F401
from .configs import C1, C2, C3, C4, C5, CONFIGS, StageConfig, get, stage_flops, with_  # noqa: F401
