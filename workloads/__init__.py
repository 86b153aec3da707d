"""Seeded synthetic inputs for the paged-attention decode step.

Shared by the tests, the smoke check and the benchmark.  It imports neither
the oracle nor the HIP binding, and holds none of the method's arithmetic:
it draws lengths, placements and tensors, and keeps the host-side block
bookkeeping (free pool, block tables, reference counts, copy-on-write
decisions) whose outputs are the kernels' index inputs.
"""

from .blocks import BlockManager, BlockPool, OutOfBlocks
from .configs import (
    BITS_NUMPY,
    BITS_TORCH,
    CONFIG_4_ON_WRITE,
    CONFIG_5_HEAD_SCALES,
    CONFIG_6_HEAD_SCALES,
    CONFIGS,
    ELEM_BYTES,
    TORCH_DTYPE,
    PREFILL_CONFIGS,
    SCALED_FORMATS,
    Case,
    Config,
    PrefillCase,
    PrefillConfig,
    bits,
    draw_context_lens,
    make_case,
    make_prefill_case,
)

__all__ = [
    "BlockManager", "BlockPool", "OutOfBlocks", "BITS_NUMPY", "BITS_TORCH", "CONFIG_4_ON_WRITE",
    "CONFIG_5_HEAD_SCALES", "CONFIG_6_HEAD_SCALES", "CONFIGS", "ELEM_BYTES", "TORCH_DTYPE", "Case", "Config", "bits", "draw_context_lens", "make_case",
    "PREFILL_CONFIGS", "SCALED_FORMATS", "PrefillCase", "PrefillConfig", "make_prefill_case",
]
