"""Seeded synthetic inputs for decode attention over a (paged) KV cache.

This package only draws random numbers and arranges them in the storage
layouts the decode call reads (contiguous BNSD, paged block pools addressed by
a block table).  It holds none of the attention arithmetic: no dot products,
no softmax, no merging.  Both the float64 oracle tests and the GPU parity
tests / benchmark build their inputs here, so the two sides always read the
same stored bytes.
"""

from .workloads import (  # noqa: F401
    CONFIGS,
    Workload,
    make_workload,
    config_workload,
    paged_block_table,
    blocks_needed,
    DTYPES,
)
