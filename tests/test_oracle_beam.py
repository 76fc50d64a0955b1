"""Beam search on the oracle's manager.

"vLLM PagedAttention and continuous batching", section "Sharing with
reference counts and copy-on-write": beam candidates share blocks; candidates
that leave the beam drop their references and blocks at zero are released;
new candidates take new blocks only for the token they add, copying a shared
last block before writing into it.  The oracle does this with fork, free and
append (oracle.replay.beam_reorder, then the usual append).

Pins:
* brute force: every beam's logical token list (kept as plain Python lists,
  no blocks at all) equals what its table gathers from the pool, after every
  step, for random widths, block sizes and parent choices;
* invariants over the 32 steps of the beam workload: reference counts equal
  the number of table entries naming a block, free and live blocks partition
  the pool, each sequence owns the block it just wrote, every beam of a
  prompt maps the prompt's full blocks, and sharing uses fewer blocks than
  separate copies would.
"""

import numpy as np
import pytest

from oracle.cache_ops import HostPool, copy_blocks, gather, write_kv
from oracle.manager import BlockManager
from oracle.replay import OracleState, beam_reorder, build_state, manager_step
from workloads import make_workload


@pytest.mark.parametrize("seed", range(6))
def test_beam_brute_force_logical_contents(seed):
    rng = np.random.default_rng(700 + seed)
    B = int(rng.choice([1, 2, 3, 4, 8]))
    W = int(rng.integers(2, 5))
    prompts = 2
    S = prompts * W
    steps = 24
    maxb = 64
    P = 200
    mgr = BlockManager(P, B, rng.permutation(P))
    pool = HostPool(1, P, 1, B, 1)
    st = OracleState(mgr, [[-1] * maxb for _ in range(S)], [0] * S, pool, (0,))
    logical = [[] for _ in range(S)]
    marker = 1
    # prompt of each request: its first beam appends, the others fork it
    for p in range(prompts):
        root = p * W
        n = int(rng.integers(1, 3 * B + 2))
        toks = list(range(marker, marker + n))
        marker += n
        slots, pairs = mgr.append_tokens(st.tables[root], 0, n)
        copy_blocks(pool, pairs)
        vals = np.array(toks, dtype=np.uint16).reshape(n, 1, 1)
        write_kv(pool, 0, vals, vals, slots)
        st.lens[root] = n
        logical[root] = toks
        for b in range(1, W):
            child = mgr.fork(st.tables[root], n)
            st.tables[root + b][: len(child)] = child
            st.lens[root + b] = n
            logical[root + b] = list(toks)
    for step in range(steps):
        parents = np.concatenate([p * W + np.sort(rng.integers(0, W, size=W)) for p in range(prompts)])
        beam_reorder(st, parents)
        logical = [list(logical[int(par)]) for par in parents]
        slots, pairs, _ = manager_step(st)
        copy_blocks(pool, pairs)
        new = np.arange(marker, marker + S, dtype=np.uint16).reshape(S, 1, 1)
        marker += S
        write_kv(pool, 0, new, new, slots)
        for s in range(S):
            logical[s].append(int(new[s, 0, 0]))
        for s in range(S):
            Kc, Vc = gather(pool, 0, st.tables[s], st.lens[s])
            assert Kc[:, 0, 0].tolist() == logical[s], (B, W, step, s)
            assert Vc[:, 0, 0].tolist() == logical[s]
        # every referenced block is counted once per table entry; nothing leaks
        live = {}
        for t, n in zip(st.tables, st.lens):
            for blk in t[: -(-n // B)]:
                live[blk] = live.get(blk, 0) + 1
        assert all(mgr.ref[b] == live.get(b, 0) for b in range(P))
        assert len(mgr.free_list()) + len(live) == P


def test_beam_workload_invariants_and_savings():
    wl = make_workload(6)
    c = wl.cfg
    B, W = c.B, c.branches
    st = build_state(wl, maxb=wl.max_blocks(c.steps))
    prompt_len = [st.lens[p * W] for p in range(c.prompts)]
    prompt_blocks = [list(st.tables[p * W][: n // B]) for p, n in enumerate(prompt_len)]
    copies = 0
    for step in range(c.steps):
        beam_reorder(st, wl.parents(step))
        _, pairs, lens = manager_step(st)
        copies += len(pairs)
        refs = {}
        for t, n in zip(st.tables, st.lens):
            for blk in t[: -(-n // B)]:
                refs[blk] = refs.get(blk, 0) + 1
        assert all(st.mgr.ref[b] == refs.get(b, 0) for b in range(wl.P))
        free = st.mgr.free_list()
        assert len(free) + len(refs) == wl.P and not set(free) & set(refs)
        for s, (t, n) in enumerate(zip(st.tables, st.lens)):
            last = t[(n - 1) // B]
            assert st.mgr.ref[last] == 1, (step, s)           # the block just written is private
            pb = prompt_blocks[s // W]
            assert list(t[: len(pb)]) == pb                    # the prompt's full blocks stay shared
        # sharing: fewer live blocks than every beam holding its own copy
        separate = sum(-(-n // B) for n in st.lens)
        assert len(refs) < separate
    assert copies > 0
