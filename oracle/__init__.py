"""CPU oracle for the stage-task path -- TEST INFRASTRUCTURE, not product code.

A plain, slow, float64 NumPy statement of what one stage task computes (one DiT
Transformer block at one denoising step for one latent chunk, reading the noisy
KV that earlier chunks left at that same step), of the patch embedding and
output head either side of the block stack, and of the two chunk x step
schedules (sequential, staggered).  It shares no code with the HIP path; only
the seeded generators in ``synthetic`` serve both.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The product path never routes through it.

Parity status: every function is pinned by a ``-m "not gpu"`` test against a
closed form, a library routine, brute force or an invariant (see
``tests/test_oracle_*.py``).  The absolute values of a whole block are fixed
only by the readings taken where the pages are silent (block layout,
normalisation, modulation, RoPE split, precisions), which the docstrings of
``block.py`` and ``head.py`` state; the pages print no worked numeric example
of the block.
"""
from .block import (  # noqa: F401
    adaln, attention, block_task, context_kv, cross_q, ffn_hidden, gelu_tanh, layer_norm,
    modulation, qkv_phase, qkv_proj, residual, rest_phase, rope3d, rope_segments, silu, sinusoid,
    time_embedding, token_positions,
)
from .head import output_head, patch_embed, patchify, time_mlp, unpatchify  # noqa: F401
from .schedule import RingPool, run_schedule, shifted_timesteps, staggered_ticks  # noqa: F401
