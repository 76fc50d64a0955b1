"""Paged key/value cache and decode attention for AMD MI355X (gfx950).

Python binding of the C ABI in ``include/pa.h`` (``libpa.so``).  The binding
only marshals arguments: the pool, the block manager and every device
operation run in the native library.  PyTorch supplies device memory and
streams.
"""

from ._abi import OutOfBlocks, PAError, PA_BF16, PA_F16  # noqa: F401
from .pool import Pool, decode_workspace, dtype_code, multi_query_workspace  # noqa: F401

__all__ = ["Pool", "PAError", "OutOfBlocks", "decode_workspace", "multi_query_workspace", "dtype_code", "PA_F16",
           "PA_BF16"]
