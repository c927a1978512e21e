"""Float64 CPU oracle for FlashBlock's block-diffusion attention step.

TEST INFRASTRUCTURE ONLY: ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` are its only users.  It shares no code
with the HIP path and imports nothing from it.
"""
from .flashblock import (ALWAYS, GAMMA, GAMMA_GROUP, TAU, TAU_CUM, BlockResult, HeadState, StepData, attend,
                         cosine, decide, default_scale, external, internal_merge, merge,
                         run_block, run_block_sparse, run_blocks, SPARSE_TILE, tile_rows)

__all__ = ["ALWAYS", "GAMMA", "GAMMA_GROUP", "TAU", "TAU_CUM", "BlockResult", "HeadState", "StepData", "attend",
           "cosine", "decide", "default_scale", "external", "internal_merge", "merge",
           "run_block", "run_block_sparse", "run_blocks", "SPARSE_TILE", "tile_rows"]
