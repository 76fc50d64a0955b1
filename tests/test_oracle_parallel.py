"""oracle.parallel runs oracle.decode.decode_one in worker processes; its
layer decode must equal the single-process oracle bit for bit (the same
function on the same data), for any worker count and sequence subset."""

import numpy as np
import pytest

from oracle.cache_ops import HostPool
from oracle.decode import decode_layer
from oracle.parallel import OraclePool, default_workers
from workloads import normal_bits


def _layer(rng, S, Hq, Hkv, B, P, dtype):
    K = normal_bits(rng, (P, Hkv, B, 128), dtype)
    V = normal_bits(rng, (P, Hkv, B, 128), dtype)
    lens = [int(x) for x in rng.integers(0, 6 * B, size=S)]
    perm = rng.permutation(P)
    tables, nxt = [], 0
    for n in lens:
        nb = -(-n // B)
        tables.append(list(perm[nxt:nxt + nb]) + [10 ** 6] * (8 - nb))
        nxt += nb
    q = normal_bits(rng, (S, Hq, 128), dtype)
    return K, V, q, tables, lens


@pytest.mark.parametrize("workers,dtype", [(1, "f16"), (3, "bf16")])
def test_parallel_layer_equals_single_process(workers, dtype):
    rng = np.random.default_rng(77 + workers)
    S, Hq, Hkv, B, P = 11, 8, 2, 16, 80
    K, V, q, tables, lens = _layer(rng, S, Hq, Hkv, B, P, dtype)
    ref = decode_layer(HostPool.from_arrays(K[None], V[None]), 0, q, tables, lens, 0.0883883, dtype)
    with OraclePool(workers) as pool:
        k, v = pool.layer_buffer(K.shape)
        k[:] = K
        v[:] = V
        out, wall, busy = pool.decode_layer(q, tables, lens, 0.0883883, dtype)
        assert np.array_equal(out, ref)
        assert wall > 0 and busy > 0
        sub = [1, 4, 9]
        out2, _, _ = pool.decode_layer(q, tables, lens, 0.0883883, dtype, seqs=sub)
        assert np.array_equal(out2[sub], ref[sub])
        assert not np.any(out2[[s for s in range(S) if s not in sub]])


def test_default_workers_positive():
    assert default_workers() >= 1
