"""One GPU's share of a workload when its heads are split over several GPUs.

"vLLM PagedAttention and continuous batching", section on several GPUs: with
the heads split over GPUs every GPU keeps the same block ids and tables and
stores only its own heads of every block.  The shard therefore keeps the
sequences, the lengths, the manager history and the pool size, and divides
the query and key/value head counts by the shard count (a query group stays
with its key/value head).
"""

import numpy as np
import pytest

from workloads import make_workload


@pytest.mark.parametrize("n", [2, 4, 8])
def test_shard_keeps_sequences_and_divides_heads(n):
    base = make_workload(3)
    wl = make_workload(3, head_shards=n)
    c = wl.cfg
    assert (c.Hq, c.Hkv) == (base.cfg.Hq // n, base.cfg.Hkv // n)
    assert c.Hq // c.Hkv == base.cfg.Hq // base.cfg.Hkv
    assert c.name.endswith(f"_heads1of{n}")
    assert np.array_equal(wl.lengths0, base.lengths0)
    assert wl.history == base.history
    assert wl.P == base.P
    assert np.array_equal(wl.free_order, base.free_order)
    assert wl.q_bits(0, 0).shape == (wl.S, c.Hq, c.d)
    assert wl.knew_bits(0, 0).shape == (wl.S, c.Hkv, c.d)


def test_shard_count_must_divide_kv_heads():
    with pytest.raises(ValueError):
        make_workload(3, head_shards=3)
    with pytest.raises(ValueError):
        make_workload(3, head_shards=16)


def test_one_shard_is_the_workload():
    a, b = make_workload(1), make_workload(1, head_shards=1)
    assert a.cfg == b.cfg
    assert np.array_equal(a.q_bits(0, 0), b.q_bits(0, 0))
