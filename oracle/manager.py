"""Block manager: physical blocks, per-sequence block tables, refcounts,
fork / append / free and copy-on-write.  Pure Python.

Sources ("vLLM PagedAttention and continuous batching"):
  * section "PagedAttention: fixed blocks, non-contiguous physical memory":
    a block table maps each logical block of a sequence to a physical block;
    logical blocks fill left to right; a new physical block is taken only when
    the previous one is full (the seven-token example: two blocks after a
    seven-token prefill at block size 4, the eighth token goes into the spare
    slot, a third block only for the ninth).
  * section "Sharing with reference counts and copy-on-write": every
    physical block has a reference count; writing into a block whose count is
    above one takes a new block, copies that single block and decrements the
    old count, and the other sharers keep the original; a block whose count
    reaches zero is released; the policies are fork, append and free.
  * "PagedAttention and Online Inference", section 3: copy-on-write protects a
    shared partially filled block; reclamation must not reuse an address that
    is still referenced.

Readings where the pages are silent:
  * Free-list order: a FIFO queue seeded with a given permutation of the pool;
    allocation takes the head, release appends at the tail.
  * Several sharers writing the same shared block in one step: sequences are
    processed in batch order; each writer that sees count > 1 copies; the
    writer that finds count == 1 writes in place and keeps the original.
  * Position of the appended token: a sequence holding n tokens writes the
    new token at position n, slot = phys * B + (n mod B).
"""

from __future__ import annotations

from collections import deque
from dataclasses import dataclass
from typing import Deque, List, Optional, Sequence, Tuple


class ManagerError(Exception):
    pass


class OutOfBlocks(ManagerError):
    """Raised when no free block is left.  For multi-token or batch appends,
    ``n_done`` tells how many appends completed (and stay applied) before the
    failing one, which itself changed nothing."""

    n_done: int = 0


class InvalidArg(ManagerError):
    pass


@dataclass
class Counters:
    allocs: int = 0
    cows: int = 0
    releases: int = 0
    live_high_water: int = 0


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int,
                 free_order: Optional[Sequence[int]] = None):
        if num_blocks <= 0 or block_size <= 0:
            raise InvalidArg("pool and block size must be positive")
        order = list(range(num_blocks)) if free_order is None else [int(x) for x in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise InvalidArg("free order must be a permutation of the pool")
        self.P = num_blocks
        self.B = block_size
        self.free: Deque[int] = deque(order)
        self.ref: List[int] = [0] * num_blocks
        self.counters = Counters()

    # ---- single-block primitives ------------------------------------------
    def num_free(self) -> int:
        return len(self.free)

    def alloc(self) -> int:
        if not self.free:
            raise OutOfBlocks("no free physical block")
        blk = self.free.popleft()
        self.ref[blk] = 1
        self.counters.allocs += 1
        live = self.P - len(self.free)
        self.counters.live_high_water = max(self.counters.live_high_water, live)
        return blk

    def _check(self, blk: int) -> None:
        if not (0 <= blk < self.P):
            raise InvalidArg(f"block {blk} outside the pool")

    def incref(self, blk: int) -> None:
        self._check(blk)
        if self.ref[blk] == 0:
            raise InvalidArg(f"block {blk} is free")
        self.ref[blk] += 1

    def decref(self, blk: int) -> None:
        self._check(blk)
        if self.ref[blk] == 0:
            raise InvalidArg(f"block {blk} is already free")
        self.ref[blk] -= 1
        if self.ref[blk] == 0:
            self.free.append(blk)
            self.counters.releases += 1

    # ---- sequence-level policies --------------------------------------------
    def append_slot(self, table: List[int], n_before: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Reserve the slot of token position ``n_before`` in ``table`` (edited
        in place).  Returns (slot, cow_pair or None).  On OutOfBlocks nothing
        changes."""
        if n_before < 0:
            raise InvalidArg("negative length")
        idx, off = divmod(n_before, self.B)
        if idx >= len(table):
            raise InvalidArg("block table too short")
        if off == 0:
            blk = self.alloc()
            table[idx] = blk
            return blk * self.B, None
        last = table[idx]
        self._check(last)
        if self.ref[last] == 0:
            raise InvalidArg(f"table maps free block {last}")
        if self.ref[last] > 1:
            new = self.alloc()
            self.decref(last)
            table[idx] = new
            self.counters.cows += 1
            return new * self.B + off, (last, new)
        return last * self.B + off, None

    def append_tokens(self, table: List[int], n_before: int, count: int
                      ) -> Tuple[List[int], List[Tuple[int, int]]]:
        """``count`` successive appends starting at position ``n_before``."""
        slots: List[int] = []
        pairs: List[Tuple[int, int]] = []
        for i in range(count):
            try:
                slot, pair = self.append_slot(table, n_before + i)
            except OutOfBlocks as e:
                e.n_done = i
                raise
            slots.append(slot)
            if pair is not None:
                pairs.append(pair)
        return slots, pairs

    def append_batch(self, tables: List[List[int]], n_before: Sequence[int]
                     ) -> Tuple[List[int], List[Tuple[int, int]]]:
        """One decode step: every sequence appends one token, in batch order."""
        slots: List[int] = []
        pairs: List[Tuple[int, int]] = []
        for i, (table, n) in enumerate(zip(tables, n_before)):
            try:
                slot, pair = self.append_slot(table, int(n))
            except OutOfBlocks as e:
                e.n_done = i
                raise
            slots.append(slot)
            if pair is not None:
                pairs.append(pair)
        return slots, pairs

    def fork(self, parent_table: Sequence[int], n_tokens: int) -> List[int]:
        """A child that maps the parent's first ceil(n_tokens / B) blocks."""
        nb = -(-int(n_tokens) // self.B)
        child = list(parent_table[:nb])
        if len(child) != nb:
            raise InvalidArg("parent table too short")
        for blk in child:
            self._check(blk)
            if self.ref[blk] == 0:
                raise InvalidArg(f"parent maps free block {blk}")
        for blk in child:
            self.ref[blk] += 1
        return child

    def free_seq(self, table: Sequence[int], n_tokens: int) -> None:
        """Drop one reference to each of the sequence's ceil(n / B) blocks."""
        nb = -(-int(n_tokens) // self.B)
        blocks = list(table[:nb])
        if len(blocks) != nb:
            raise InvalidArg("table too short")
        need = {}
        for blk in blocks:
            self._check(blk)
            need[blk] = need.get(blk, 0) + 1
        for blk, k in need.items():
            if self.ref[blk] < k:
                raise InvalidArg(f"block {blk} has fewer references than the table holds")
        for blk in blocks:
            self.decref(blk)

    def free_list(self) -> List[int]:
        return list(self.free)
