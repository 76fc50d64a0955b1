"""The oracle's decode of whole layers spread over the host's cores -- TEST
INFRASTRUCTURE ONLY (used by tests/ and the cpu_baseline leg of bench.py).

No arithmetic of its own: every (layer, sequence) result is
``oracle.decode.decode_one`` -- gather the sequence's blocks by its table,
widen to float64, dense attention -- run in a worker process.  Sequences are
independent ("PagedAttention and Online Inference", verification plan item 1:
outputs are checked against a contiguous-K/V baseline), so splitting a layer
by sequence changes nothing in any result.

Workers are fresh interpreters (spawn), each limited to one BLAS thread.
Create the pool before the calling process initialises a GPU: the workers
then start from a process that has not touched it.  A layer's key and value
slabs reach the workers through a memory-mapped file (in /dev/shm when it has
room), written once by the caller.
"""

from __future__ import annotations

import os
import tempfile
import time
from typing import Optional, Sequence, Tuple

import numpy as np

_THREAD_VARS = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS")


def default_workers() -> int:
    """Cores this process may run on (its affinity mask), capped by
    OMP_NUM_THREADS when that names the process's share of a larger host."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def _init_worker():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except ImportError:
        pass


_maps = {}


def _slabs(path: str, shape: Tuple[int, ...]):
    """Read-only views of the (K, V) slabs in ``path`` (cached per worker)."""
    key = (path, shape)
    if key not in _maps:
        _maps.clear()
        mm = np.memmap(path, dtype=np.uint16, mode="r", shape=(2,) + shape)
        _maps[key] = mm
    mm = _maps[key]
    return mm[0], mm[1]


def _decode_chunk(args):
    from .cache_ops import HostPool
    from .decode import decode_one
    path, shape, dtype, scale, items = args
    K, V = _slabs(path, shape)
    pool = HostPool.from_arrays(K[None], V[None])
    out = []
    t0 = time.perf_counter()
    for s, q_bits, table, n in items:
        out.append((s, decode_one(pool, 0, q_bits, table, n, scale, dtype)))
    return out, time.perf_counter() - t0


class OraclePool:
    """A pool of spawned worker processes for the oracle's layer decode."""

    def __init__(self, workers: Optional[int] = None):
        import multiprocessing as mp
        self.workers = workers or default_workers()
        saved = {k: os.environ.get(k) for k in _THREAD_VARS}
        try:
            for k in _THREAD_VARS:
                os.environ[k] = "1"
            self._pool = mp.get_context("spawn").Pool(self.workers, initializer=_init_worker)
        finally:
            for k, v in saved.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
        self._dir = _scratch_dir()
        self._path = None
        self._mm = None

    # -- a layer's slabs -------------------------------------------------------
    def layer_buffer(self, shape: Tuple[int, ...]) -> Tuple[np.ndarray, np.ndarray]:
        """Writable (K, V) arrays of ``shape`` ([P][Hkv][B][d] uint16) that
        the next decode_layer call reads; valid until the next call of this
        method or close()."""
        self._release()
        fd, self._path = tempfile.mkstemp(prefix="pa_oracle_", suffix=".u16", dir=self._dir)
        os.close(fd)
        self._mm = np.memmap(self._path, dtype=np.uint16, mode="w+", shape=(2,) + tuple(shape))
        self._shape = tuple(shape)
        return self._mm[0], self._mm[1]

    def decode_layer(self, q_bits: np.ndarray, tables: Sequence[Sequence[int]], lens: Sequence[int],
                     scale: float, dtype: str, seqs: Optional[Sequence[int]] = None):
        """Oracle outputs [S][Hq][d] float64 (rows outside ``seqs`` stay
        zero) for the slabs last written through layer_buffer.  Returns
        (out, wall seconds of the parallel decode, summed worker seconds)."""
        if self._mm is None:
            raise RuntimeError("layer_buffer() first")
        self._mm.flush()
        S = len(lens)
        seqs = list(range(S)) if seqs is None else list(seqs)
        # longest first, dealt to chunks round-robin: balanced work per task
        order = sorted(seqs, key=lambda s: -int(lens[s]))
        nchunks = min(len(order), 4 * self.workers)
        chunks = [[] for _ in range(max(nchunks, 1))]
        for i, s in enumerate(order):
            chunks[i % len(chunks)].append((s, q_bits[s], list(map(int, tables[s])), int(lens[s])))
        tasks = [(self._path, self._shape, dtype, float(scale), c) for c in chunks if c]
        out = np.zeros(q_bits.shape, dtype=np.float64)
        t0 = time.perf_counter()
        results = self._pool.map(_decode_chunk, tasks, chunksize=1)
        wall = time.perf_counter() - t0
        busy = 0.0
        for res, secs in results:
            busy += secs
            for s, o in res:
                out[s] = o
        return out, wall, busy

    def _release(self):
        if self._mm is not None:
            del self._mm
            self._mm = None
        if self._path is not None:
            try:
                os.unlink(self._path)
            except OSError:
                pass
            self._path = None

    def close(self):
        self._release()
        if self._pool is not None:
            self._pool.close()
            self._pool.join()
            self._pool = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def _scratch_dir() -> str:
    """/dev/shm when it exists and has room for a few large layers, else the
    temporary directory."""
    try:
        st = os.statvfs("/dev/shm")
        if st.f_bavail * st.f_frsize >= (8 << 30):
            return "/dev/shm"
    except OSError:
        pass
    return tempfile.gettempdir()
