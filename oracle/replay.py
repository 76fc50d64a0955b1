"""Replay a workload's abstract history and decode steps on the oracle's own
manager and host pool.

The workload object supplies only inputs (lengths, pool size, free order,
history ops, seeded values); every table, slot, copy-on-write pair and cache
write below is computed here by the oracle.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import numpy as np

from .cache_ops import HostPool, copy_blocks, write_kv
from .decode import decode_layer
from .manager import BlockManager


@dataclass
class OracleState:
    mgr: BlockManager
    tables: List[List[int]]
    lens: List[int]
    pool: Optional[HostPool]
    layers: Tuple[int, ...]        # workload layer held at each pool layer index


def build_state(wl, layers: Sequence[int] = (), maxb: Optional[int] = None,
                fill_bits: int = 0) -> OracleState:
    """Run the history.  With ``layers`` empty only the manager runs; else
    prefill values of those workload layers are written into a host pool
    whose other slots hold ``fill_bits``."""
    c = wl.cfg
    maxb = wl.max_blocks() if maxb is None else maxb
    mgr = BlockManager(wl.P, c.B, wl.free_order)
    tables = [[-1] * maxb for _ in range(wl.S)]
    lens = [0] * wl.S
    pool = HostPool(len(layers), wl.P, c.Hkv, c.B, c.d, fill_bits) if layers else None
    for op_index, op in enumerate(wl.history):
        if op[0] == "append":
            _, s, ntok = op
            slots, pairs = mgr.append_tokens(tables[s], lens[s], ntok)
            if pool is not None:
                copy_blocks(pool, pairs)
                for li, layer in enumerate(layers):
                    write_kv(pool, li, wl.prefill_bits(layer, op_index, ntok, "k"),
                             wl.prefill_bits(layer, op_index, ntok, "v"), slots)
            lens[s] += ntok
        elif op[0] == "fork":
            _, child, parent, ntok = op
            shared = mgr.fork(tables[parent], ntok)
            tables[child][: len(shared)] = shared
            lens[child] = ntok
        else:
            raise ValueError(op)
    return OracleState(mgr, tables, lens, pool, tuple(layers))


def manager_step(st: OracleState) -> Tuple[List[int], List[Tuple[int, int]], List[int]]:
    """Every sequence appends one token (batch order).  Returns (slots, cow
    pairs, context lengths after the step)."""
    slots, pairs = st.mgr.append_batch(st.tables, st.lens)
    st.lens = [n + 1 for n in st.lens]
    return slots, pairs, list(st.lens)


def beam_reorder(st: OracleState, parents: Sequence[int]) -> None:
    """Beam selection before a step ("vLLM PagedAttention and continuous
    batching", section "Sharing with reference counts and copy-on-write"):
    each new sequence forks the old sequence it continues (one more reference
    to each of its blocks), then every old sequence is freed (one fewer;
    blocks reaching zero are released).  Shared last blocks are copied at the
    next append, by the usual rule."""
    maxb = len(st.tables[0]) if st.tables else 0
    new_tables, new_lens = [], []
    for par in parents:
        par = int(par)
        child = st.mgr.fork(st.tables[par], st.lens[par])
        new_tables.append(child + [-1] * (maxb - len(child)))
        new_lens.append(st.lens[par])
    for table, n in zip(st.tables, st.lens):
        st.mgr.free_seq(table, n)
    st.tables, st.lens = new_tables, new_lens


def decode_step(st: OracleState, wl, step: int = 0) -> Tuple[np.ndarray, List[int], List[Tuple[int, int]]]:
    """Manager step, block copies, per-layer write of the new token and dense
    attention.  Returns (out [len(layers)][S][Hq][d] float64, slots, pairs)."""
    c = wl.cfg
    slots, pairs, lens = manager_step(st)
    copy_blocks(st.pool, pairs)
    outs = []
    for li, layer in enumerate(st.layers):
        write_kv(st.pool, li, wl.knew_bits(layer, step), wl.vnew_bits(layer, step), slots)
        outs.append(decode_layer(st.pool, li, wl.q_bits(layer, step), st.tables, lens,
                                 float(wl.scale), c.dtype))
    return np.stack(outs), slots, pairs
