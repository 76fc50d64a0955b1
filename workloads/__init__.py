"""Seeded synthetic inputs for paged decode attention.

This package is shared by the HIP path's callers (tests, bench) and by the
CPU oracle's callers.  It holds only input generation: the five workload
shapes, their seeded random draws (lengths, pool permutations, query/key/value
values rounded to the storage dtype) and the abstract sequence history each
workload starts from.  It contains none of the method's arithmetic: no
attention, no block-table bookkeeping, no cache scatter or copy.
"""

from .configs import CONFIGS, DecodeConfig, get_config  # noqa: F401
from .gen import (  # noqa: F401
    Workload,
    make_workload,
    with_headroom,
    rng_for,
    round_to_dtype_bits,
    normal_bits,
    dtype_nan_bits,
)
