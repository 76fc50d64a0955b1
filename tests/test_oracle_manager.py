"""Pins of oracle.manager: the seven-token example and the refcount /
copy-on-write rules of the NetLeverage article, the allocation counts of the
five-length worked example, and invariants checked over random op traces."""

import numpy as np
import pytest

from oracle import accounting as A
from oracle.manager import BlockManager, InvalidArg, OutOfBlocks
from oracle.replay import build_state, manager_step
from tests.conftest import load_golden
from workloads import make_workload


def test_seven_token_example():
    g = load_golden("seven_token_example.json")
    B = g["block_size_reading"]
    m = BlockManager(16, B)
    table = [-1] * 8
    slots, pairs = m.append_tokens(table, 0, g["prefill_tokens"])
    used = lambda: sum(1 for b in table if b >= 0)
    assert used() == g["logical_blocks_after_prefill"]
    assert pairs == []
    allocs_before = m.counters.allocs
    slot8, pair = m.append_slot(table, g["prefill_tokens"])        # 8th token
    assert (m.counters.allocs > allocs_before) == g["next_token_takes_new_block"]
    assert slot8 == table[1] * B + 3 and pair is None
    slot9, _ = m.append_slot(table, g["prefill_tokens"] + 1)       # 9th token
    assert (m.counters.allocs > allocs_before) == g["token_after_spare_slot_takes_new_block"]
    assert used() == g["logical_blocks_at_end"]
    assert slot9 == table[2] * B
    # logical blocks fill left to right: token t sits in logical block t // B
    assert [s // B for s in slots] == [table[t // B] for t in range(7)]


def test_fifo_free_list_and_release():
    m = BlockManager(4, 2, free_order=[2, 0, 3, 1])
    a, b = m.alloc(), m.alloc()
    assert (a, b) == (2, 0)
    m.decref(a)                      # released to the tail
    assert m.free_list() == [3, 1, 2]
    assert m.alloc() == 3 and m.alloc() == 1 and m.alloc() == 2
    with pytest.raises(OutOfBlocks):
        m.alloc()
    with pytest.raises(InvalidArg):
        BlockManager(3, 2, free_order=[0, 0, 1])


def test_double_free_and_free_block_incref_rejected():
    m = BlockManager(4, 2)
    b = m.alloc()
    m.decref(b)
    with pytest.raises(InvalidArg):
        m.decref(b)
    with pytest.raises(InvalidArg):
        m.incref(b)
    with pytest.raises(InvalidArg):
        m.decref(99)


def test_copy_on_write_shared_partial_block():
    B = 4
    m = BlockManager(8, B, free_order=list(range(8)))
    parent = [-1] * 4
    m.append_tokens(parent, 0, 6)                # blocks 0, 1; block 1 has 2 tokens
    child = m.fork(parent, 6) + [-1, -1]
    assert m.ref[0] == 2 and m.ref[1] == 2
    # parent writes token 6 into shared block 1 (count 2): copy
    slot, pair = m.append_slot(parent, 6)
    assert pair == (1, 2) and parent[1] == 2 and slot == 2 * B + 2
    assert m.ref[1] == 1 and m.ref[2] == 1
    assert child[:2] == [0, 1]                   # the sharer keeps the original
    # child now finds count 1: writes in place
    slot, pair = m.append_slot(child, 6)
    assert pair is None and slot == 1 * B + 2
    # full shared block: the next token opens a new block, no copy
    parent2 = [-1] * 4
    m2 = BlockManager(8, B)
    m2.append_tokens(parent2, 0, 8)
    kid = m2.fork(parent2, 8) + [-1, -1]
    slot, pair = m2.append_slot(kid, 8)
    assert pair is None and kid[2] == 2 and m2.ref[0] == 2 and m2.ref[1] == 2


def test_exhaustion_leaves_state_unchanged():
    B = 2
    m = BlockManager(2, B)
    t1, t2 = [-1] * 4, [-1] * 4
    m.append_tokens(t1, 0, 3)                    # both blocks used
    m.fork(t1, 3)
    snapshot = (list(m.ref), m.free_list(), list(t1), m.counters.allocs)
    with pytest.raises(OutOfBlocks):
        m.append_slot(t1, 3)                     # CoW would need a block
    with pytest.raises(OutOfBlocks) as e:
        m.append_tokens(t2, 0, 5)
    assert e.value.n_done == 0
    assert (list(m.ref), m.free_list(), list(t1), m.counters.allocs) == snapshot


def _invariants(m: BlockManager, tables, lens):
    live = {}
    for t, n in zip(tables, lens):
        for blk in t[: A.blocks_needed(n, m.B)]:
            live[blk] = live.get(blk, 0) + 1
    assert sum(m.ref) == sum(live.values())
    for blk in range(m.P):
        assert m.ref[blk] == live.get(blk, 0)
    free = m.free_list()
    assert len(free) == len(set(free))
    assert len(free) + sum(1 for r in m.ref if r > 0) == m.P
    assert all(m.ref[b] == 0 for b in free)


@pytest.mark.parametrize("seed", range(6))
def test_random_traces_keep_invariants(seed):
    rng = np.random.default_rng(seed)
    P, B, maxb = int(rng.integers(2, 9)), int(rng.choice([1, 2, 4])), 12
    m = BlockManager(P, B, free_order=rng.permutation(P))
    tables, lens = [], []
    for _ in range(300):
        op = rng.integers(0, 4)
        try:
            if op == 0 or not tables:
                t = [-1] * maxb
                n = int(rng.integers(0, 3 * B))
                m.append_tokens(t, 0, n)
                tables.append(t)
                lens.append(n)
            elif op == 1:
                i = int(rng.integers(len(tables)))
                if lens[i] < maxb * B:
                    m.append_slot(tables[i], lens[i])
                    lens[i] += 1
            elif op == 2:
                i = int(rng.integers(len(tables)))
                child = m.fork(tables[i], lens[i]) + [-1] * maxb
                tables.append(child[:maxb])
                lens.append(lens[i])
            else:
                i = int(rng.integers(len(tables)))
                m.free_seq(tables[i], lens[i])
                tables.pop(i)
                lens.pop(i)
        except OutOfBlocks as e:
            if op == 0:                      # partial prefill stays applied
                tables.append(t)
                lens.append(e.n_done)
        _invariants(m, tables, lens)


def test_five_lengths_allocate_as_the_worked_example():
    for cfg, total in ((1, 62), (2, 32)):
        wl = make_workload(cfg)
        st = build_state(wl)
        manager_step(st)
        B = wl.cfg.B
        assert [A.blocks_needed(n, B) for n in st.lens] == \
            [A.blocks_needed(n, B) for n in (37, 91, 128, 201, 511)]
        if cfg == 1:
            assert st.mgr.counters.allocs == total
            # table = the first 62 entries of the free-order permutation, in order
            flat = [b for t, n in zip(st.tables, st.lens) for b in t[: A.blocks_needed(n, B)]]
            assert flat == list(wl.free_order[:total])


def test_config2_one_cow_into_shared_prefix_block():
    wl = make_workload(2)
    st = build_state(wl)
    p0, p1 = st.tables[1][0], st.tables[1][1]
    assert st.tables[0][:2] == st.tables[2][:2] == st.tables[3][:2] == [p0, p1]
    assert st.mgr.ref[p0] == 4 and st.mgr.ref[p1] == 4
    slots, pairs, lens = manager_step(st)
    assert len(pairs) == 1 and pairs[0][0] == p1
    new = pairs[0][1]
    assert st.tables[0][:2] == [p0, new]
    assert slots[0] == new * 32 + 36 % 32
    assert st.mgr.ref[p1] == 3
    assert st.tables[1][:2] == st.tables[2][:2] == st.tables[3][:2] == [p0, p1]


def test_config5_first_step_three_of_four_branches_copy():
    wl = make_workload(5)
    st = build_state(wl)
    _, pairs, _ = manager_step(st)
    prompts = wl.lengths0[:: wl.cfg.branches] - 1
    partial = int(np.sum(prompts % wl.cfg.B != 0))
    assert len(pairs) == 3 * partial
    for p in range(wl.cfg.prompts):
        root = 4 * p
        n = int(prompts[p])
        nb = A.blocks_needed(n, 16)
        if n % 16:
            last_orig = [pr for pr in pairs if pr[1] == st.tables[root][nb - 1]]
            assert len(last_orig) == 1
            # branch 3 kept the original block in place
            assert st.tables[root + 3][nb - 1] == last_orig[0][0]
            assert st.mgr.ref[last_orig[0][0]] == 1
