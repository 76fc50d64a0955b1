"""Several new tokens per sequence (chunked prefill, speculative verification)
on the oracle.

oracle.decode.multi_query_one: query t of nq sits at position n - nq + t and
attends to positions 0 .. n - nq + t.  Pins, each independent of its code:
* one query is decode_one exactly;
* sequential equivalence: the nq outputs equal those of nq one-token decode
  steps, each appending its token through the oracle's manager and cache
  write and attending over the cache as it then stands (the point of a
  chunked prefill or of verifying draft tokens: the same result as taking
  the tokens one at a time);
* a library routine: PyTorch's scaled_dot_product_attention in float64 on
  the CPU with an explicit position mask;
* a planted top-left alignment of the mask (query t sees t + 1 positions)
  fails the pins.
"""

import numpy as np
import pytest

from oracle.cache_ops import HostPool, write_kv
from oracle.decode import decode_one, multi_query_one
from oracle.dtypes import bits_to_f64
from oracle.manager import BlockManager
from workloads import round_to_dtype_bits

torch = pytest.importorskip("torch")


def _seq(rng, n, B, Hkv, d, dtype, P=None):
    P = P or -(-n // B) + 4
    mgr = BlockManager(P, B, rng.permutation(P))
    pool = HostPool(1, P, Hkv, B, d)
    table = [-1] * (-(-n // B) + 2)
    slots, _ = mgr.append_tokens(table, 0, n)
    k = round_to_dtype_bits(rng.standard_normal((n, Hkv, d)).astype(np.float32), dtype)
    v = round_to_dtype_bits(rng.standard_normal((n, Hkv, d)).astype(np.float32), dtype)
    write_kv(pool, 0, k, v, slots)
    return mgr, pool, table, k, v


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_one_query_is_decode(dtype):
    rng = np.random.default_rng(1)
    mgr, pool, table, _, _ = _seq(rng, 77, 16, 2, 128, dtype)
    q = round_to_dtype_bits(rng.standard_normal((1, 8, 128)).astype(np.float32), dtype)
    got = multi_query_one(pool, 0, q, table, 77, 0.088, dtype)
    assert np.array_equal(got[0], decode_one(pool, 0, q[0], table, 77, 0.088, dtype))


@pytest.mark.parametrize("n0,nq,B,G", [(40, 7, 16, 4), (0, 20, 8, 1), (129, 33, 32, 2), (5, 1, 4, 8)])
def test_sequential_equivalence(n0, nq, B, G):
    """nq tokens at once == nq decode steps one token at a time."""
    rng = np.random.default_rng(100 + n0 + nq)
    dtype, Hkv, d = "f16", 2, 128
    Hq = G * Hkv
    n = n0 + nq
    P = -(-n // B) + 3
    k = round_to_dtype_bits(rng.standard_normal((n, Hkv, d)).astype(np.float32), dtype)
    v = round_to_dtype_bits(rng.standard_normal((n, Hkv, d)).astype(np.float32), dtype)
    q = round_to_dtype_bits(rng.standard_normal((nq, Hq, d)).astype(np.float32), dtype)
    order = rng.permutation(P)
    # one token at a time
    mgr = BlockManager(P, B, order)
    pool = HostPool(1, P, Hkv, B, d)
    table = [-1] * P
    if n0:
        slots, _ = mgr.append_tokens(table, 0, n0)
        write_kv(pool, 0, k[:n0], v[:n0], slots)
    steps = []
    for t in range(nq):
        slot, _ = mgr.append_slot(table, n0 + t)
        write_kv(pool, 0, k[n0 + t: n0 + t + 1], v[n0 + t: n0 + t + 1], [slot])
        steps.append(decode_one(pool, 0, q[t], table, n0 + t + 1, 0.09, dtype))
    # all at once, from a fresh manager with the same free order
    mgr2 = BlockManager(P, B, order)
    pool2 = HostPool(1, P, Hkv, B, d)
    table2 = [-1] * P
    slots, _ = mgr2.append_tokens(table2, 0, n)
    write_kv(pool2, 0, k, v, slots)
    got = multi_query_one(pool2, 0, q, table2, n, 0.09, dtype)
    assert np.array_equal(got, np.stack(steps))


@pytest.mark.parametrize("nq,G", [(9, 4), (1, 2), (31, 1)])
def test_matches_torch_sdpa_with_position_mask(nq, G):
    rng = np.random.default_rng(7 + nq)
    dtype, Hkv, d, B, n = "bf16", 2, 128, 16, 150
    Hq = G * Hkv
    mgr, pool, table, k, v = _seq(rng, n, B, Hkv, d, dtype)
    q = round_to_dtype_bits(rng.standard_normal((nq, Hq, d)).astype(np.float32), dtype)
    got = multi_query_one(pool, 0, q, table, n, 0.0883, dtype)
    Q = torch.from_numpy(bits_to_f64(q, dtype)).permute(1, 0, 2)                     # [Hq][nq][d]
    K = torch.from_numpy(bits_to_f64(k, dtype)).permute(1, 0, 2).repeat_interleave(G, 0)
    V = torch.from_numpy(bits_to_f64(v, dtype)).permute(1, 0, 2).repeat_interleave(G, 0)
    qpos = torch.arange(n - nq, n)[:, None]
    kpos = torch.arange(n)[None, :]
    mask = kpos <= qpos                                                              # [nq][n]
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=0.0883)
    assert np.max(np.abs(got - ref.permute(1, 0, 2).numpy())) < 1e-12


def test_planted_top_left_alignment_fails():
    """A mask aligned at the top left (query t sees positions 0..t) breaks
    the sequential-equivalence pin."""
    rng = np.random.default_rng(3)
    dtype, n, nq = "f16", 60, 5
    mgr, pool, table, _, _ = _seq(rng, n, 16, 1, 128, dtype)
    q = round_to_dtype_bits(rng.standard_normal((nq, 4, 128)).astype(np.float32), dtype)
    good = multi_query_one(pool, 0, q, table, n, 0.1, dtype)
    wrong = np.stack([decode_one(pool, 0, q[t], table, t + 1, 0.1, dtype) for t in range(nq)])
    right = np.stack([decode_one(pool, 0, q[t], table, n - nq + t + 1, 0.1, dtype) for t in range(nq)])
    assert np.array_equal(good, right)
    assert not np.allclose(wrong, right)
