"""Host model of the paged K/V cache: per-layer key and value block arrays,
the slot scatter of new tokens, whole-block copies and the gather of one
sequence's blocks into contiguous keys/values.

Sources ("vLLM PagedAttention and continuous batching"):
  * "PagedAttention: fixed blocks, non-contiguous physical memory": one
    contiguous allocation sliced into physical blocks; block j of a sequence
    holds the keys and values of its j-th group of B tokens; the blocks of a
    sequence need not be adjacent.
  * "The kernel page, and what the 2023 runs measured": keys and values are
    kept in separate caches.
  * "Sharing with reference counts and copy-on-write": a copy-on-write copies
    that one block (reading taken: every slot of the block, every layer, keys
    and values).
  * "How it works": prefill and decode write each token's key and value into
    the cache.

Storage: raw 16-bit patterns (uint16) of shape [L][P][Hkv][B][d] for keys and
the same for values; a slot index is phys * B + offset.
"""

from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np


class HostPool:
    def __init__(self, L: int, P: int, Hkv: int, B: int, d: int, fill_bits: int = 0):
        self.L, self.P, self.Hkv, self.B, self.d = L, P, Hkv, B, d
        shape = (L, P, Hkv, B, d)
        self.K = np.full(shape, fill_bits, dtype=np.uint16)
        self.V = np.full(shape, fill_bits, dtype=np.uint16)

    @classmethod
    def from_arrays(cls, K: np.ndarray, V: np.ndarray) -> "HostPool":
        L, P, Hkv, B, d = K.shape
        pool = cls.__new__(cls)
        pool.L, pool.P, pool.Hkv, pool.B, pool.d = L, P, Hkv, B, d
        pool.K = K
        pool.V = V
        return pool


def write_kv(pool: HostPool, layer: int, k_new: np.ndarray, v_new: np.ndarray,
             slots: Sequence[int]) -> None:
    """Token i's key/value [Hkv][d] go to slot slots[i] of ``layer``; a
    negative slot means the token is skipped."""
    B = pool.B
    for i, slot in enumerate(slots):
        slot = int(slot)
        if slot < 0:
            continue
        blk, off = divmod(slot, B)
        pool.K[layer, blk, :, off, :] = k_new[i]
        pool.V[layer, blk, :, off, :] = v_new[i]


def copy_blocks(pool: HostPool, pairs: Sequence[Tuple[int, int]]) -> None:
    """For each (src, dst): the whole block, every layer, keys and values."""
    for src, dst in pairs:
        pool.K[:, int(dst)] = pool.K[:, int(src)]
        pool.V[:, int(dst)] = pool.V[:, int(src)]


def gather(pool: HostPool, layer: int, table: Sequence[int], n: int) -> Tuple[np.ndarray, np.ndarray]:
    """Contiguous K, V of token positions 0..n-1: [n][Hkv][d] uint16 each."""
    B = pool.B
    Kc = np.empty((n, pool.Hkv, pool.d), dtype=np.uint16)
    Vc = np.empty((n, pool.Hkv, pool.d), dtype=np.uint16)
    for t in range(n):
        blk = int(table[t // B])
        Kc[t] = pool.K[layer, blk, :, t % B, :]
        Vc[t] = pool.V[layer, blk, :, t % B, :]
    return Kc, Vc
