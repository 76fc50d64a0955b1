"""Preemption by swapping: move every block of a group of sequences to a
second pool (the host side) and back.

Source: "vLLM PagedAttention and continuous batching", section "Preemption
when blocks run out": a sequence is evicted with all of its blocks or not at
all, because a later step needs the whole prefix; sequences that share
memory (the beams of one search) are preempted and resumed together; the
evicted blocks go to CPU memory managed by a second block allocator, whose
size the design bounds by the number of GPU blocks.

Readings where the pages are silent:
  * A block moves with all of its references: its copy in the other pool gets
    as many references as the group holds, so sharing inside the group
    survives the round trip; a block also mapped by a sequence outside the
    group cannot move (the group would not own all of its references).
  * Order: new blocks are taken in order of first appearance in the group's
    tables (sequence by sequence, entry by entry); the old ones are released
    by dropping the group's references in the same order as freeing each
    sequence would.
"""

from __future__ import annotations

from typing import List, Sequence, Tuple

from .cache_ops import HostPool
from .manager import BlockManager, InvalidArg, OutOfBlocks


def move_blocks(src: BlockManager, dst: BlockManager, tables: List[List[int]],
                lens: Sequence[int]) -> List[Tuple[int, int]]:
    """Move the group's blocks from ``src`` to ``dst``; ``tables`` are
    rewritten in place.  Returns (old, new) pairs.  Nothing changes on error."""
    if src.B != dst.B:
        raise InvalidArg("pools differ in block size")
    B = src.B
    order: List[int] = []
    held = {}
    for table, n in zip(tables, lens):
        nb = -(-int(n) // B)
        if len(table) < nb:
            raise InvalidArg("table too short")
        for blk in table[:nb]:
            src._check(blk)
            if blk not in held:
                order.append(blk)
                held[blk] = 0
            held[blk] += 1
    for blk in order:
        if src.ref[blk] != held[blk]:
            raise InvalidArg(f"block {blk} is also mapped outside the group")
    if dst.num_free() < len(order):
        raise OutOfBlocks("destination pool has too few free blocks")
    new_of = {}
    pairs: List[Tuple[int, int]] = []
    for blk in order:
        new = dst.alloc()
        for _ in range(held[blk] - 1):
            dst.incref(new)
        new_of[blk] = new
        pairs.append((blk, new))
    for table, n in zip(tables, lens):
        src.free_seq(table, n)
    for table, n in zip(tables, lens):
        nb = -(-int(n) // B)
        table[:nb] = [new_of[blk] for blk in table[:nb]]
    return pairs


def copy_between(src: HostPool, dst: HostPool, pairs: Sequence[Tuple[int, int]]) -> None:
    """Whole blocks, every layer, keys and values, from one pool to the other."""
    for a, b in pairs:
        dst.K[:, int(b)] = src.K[:, int(a)]
        dst.V[:, int(b)] = src.V[:, int(a)]
