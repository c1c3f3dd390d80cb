"""Seeded synthetic inputs shared by the oracle-side tests, the GPU tests and the bench.

This package draws random numbers and lays them out in memory (page pool,
block table, segment buffers).  It holds none of the attention arithmetic:
no dot products, no softmax, no window or split rule.
"""

from .gen import (  # noqa: F401
    PagedInputs,
    SegmentInputs,
    KVWriteInputs,
    CONFIGS,
    make_paged,
    make_segments,
    make_kv_write,
    paged_config,
    segment_config,
    to_numpy_bits,
)
