"""Block size changes storage only.

"vLLM PagedAttention and continuous batching", section "PagedAttention: fixed
blocks, non-contiguous physical memory": the attention mathematics is the
same whatever the block size; blocks only decide where each position is
stored and how much of the last block is left empty.  So the same sequences,
history and values run at block sizes 8 ... 128 must give the same oracle
outputs, bit for bit (the oracle gathers each sequence into the same
contiguous arrays before the dense softmax), while the allocation counts
follow ceil(n / B).
"""

import numpy as np
import pytest

from oracle.accounting import blocks_needed
from oracle.replay import build_state, decode_step
from workloads import make_workload, with_headroom
from workloads.gen import dtype_nan_bits

SIZES = (8, 16, 32, 64, 128)


def test_override_keeps_seeds_lengths_history_and_values():
    base = make_workload(3)
    for B in SIZES:
        wl = make_workload(3, block_size=B)
        assert wl.cfg.B == B and wl.cfg.cfg_id == 3
        assert f"_b{B}_" in wl.cfg.name
        assert np.array_equal(wl.lengths0, base.lengths0)
        assert wl.history == base.history
        assert np.array_equal(wl.q_bits(5, 1), base.q_bits(5, 1))
        assert np.array_equal(wl.prefill_bits(0, 3, 7, "v"), base.prefill_bits(0, 3, 7, "v"))
        used = sum(blocks_needed(int(n), B) for n in wl.lengths0)
        assert wl.P == int(np.ceil(1.25 * used))          # the 1.25x pool rule at every B
        assert sorted(wl.free_order.tolist()) == list(range(wl.P))


def test_fixed_pool_keeps_its_ratio():
    # config 1: 64 blocks for 62 used at B=16
    for B in SIZES:
        wl = make_workload(1, block_size=B)
        used = sum(blocks_needed(int(n), B) for n in wl.lengths0)
        assert wl.P == -(-64 * used // 62)
        assert wl.P >= used


@pytest.mark.parametrize("cfg", [1, 2])
def test_oracle_outputs_identical_across_block_sizes(cfg):
    """Manager, copy-on-write, cache writes and gathers at every block size
    give the same logical cache, so the same outputs bit for bit."""
    steps = 2
    ref = None
    for B in SIZES:
        wl = with_headroom(make_workload(cfg, block_size=B), steps)
        c = wl.cfg
        st = build_state(wl, layers=tuple(range(c.L)), maxb=wl.max_blocks(steps),
                         fill_bits=dtype_nan_bits(c.dtype))
        outs = []
        for step in range(steps):
            out, slots, pairs = decode_step(st, wl, step)
            assert np.all(np.isfinite(out))
            outs.append(out)
            # every sequence's slot lies in the block its position maps to
            for s, slot in enumerate(slots):
                pos = st.lens[s] - 1
                assert slot == st.tables[s][pos // B] * B + pos % B
        outs = np.stack(outs)
        if ref is None:
            ref = outs
        else:
            assert np.array_equal(outs, ref), B


def test_config2_copy_count_depends_on_block_size():
    """Sequence 1 writes a 64-token prefix; sequence 0 maps its first
    ceil(36 / B) blocks and sequences 2, 3 the whole prefix.  For B <= 64 the
    prefix ends on a block boundary, so the history copies nothing and the
    step's write of sequence 0 at position 36 lands in a block mapped four
    times: one copy.  For B = 128 the prefix fills half of one block: the
    appends of sequences 1, 2 and 3 after it each copy that block (refcount
    4, 3, 2), leaving sequence 0 its sole owner: no copy in the step."""
    from oracle.replay import manager_step
    for B in SIZES:
        wl = make_workload(2, block_size=B)
        st = build_state(wl, maxb=wl.max_blocks(1))
        history_cows = st.mgr.counters.cows
        _, pairs, _ = manager_step(st)
        if B <= 64:
            assert (history_cows, len(pairs)) == (0, 1), B
        else:
            assert (history_cows, len(pairs)) == (3, 0), B
