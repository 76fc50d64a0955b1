"""Pins of oracle.cache_ops / oracle.decode: the slot scatter puts a token
where the gather finds it, a copy duplicates whole blocks, paging is invisible
to the result (physical block permutation), and copy-on-write isolates
sharers (the PagedAttention page's section 3 and verification plan)."""

import numpy as np

from oracle.attention import dense_attention
from oracle.cache_ops import HostPool, copy_blocks, gather, write_kv
from oracle.decode import decode_layer, decode_one
from oracle.dtypes import bf16_bits_to_f64, bits_to_f64, f16_bits_to_f64
from oracle.replay import build_state, decode_step
from workloads import make_workload, round_to_dtype_bits
from workloads.gen import dtype_nan_bits


def test_dtype_widening_exact():
    x = np.array([0.0, 1.0, -2.5, 65504.0, 6.1e-5, 1e-7], dtype=np.float32)
    assert np.array_equal(f16_bits_to_f64(x.astype(np.float16).view(np.uint16)),
                          x.astype(np.float16).astype(np.float64))
    bits = np.array([0x3F80, 0xC020, 0x0001, 0x7F7F], dtype=np.uint16)
    assert np.array_equal(bf16_bits_to_f64(bits), np.array([1.0, -2.5, 2.0 ** -133, 3.3895313892515355e38]))
    # round-to-nearest-even at the bf16 halfway point: 1 + 2^-8 -> 1.0, 1 + 3*2^-8 -> 1 + 2^-6
    y = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8], dtype=np.float32)
    assert np.array_equal(bf16_bits_to_f64(round_to_dtype_bits(y, "bf16")), [1.0, 1 + 2 ** -6])


def test_write_then_gather_roundtrip_and_skip():
    rng = np.random.default_rng(0)
    L, P, H, B, d = 2, 6, 2, 4, 8
    pool = HostPool(L, P, H, B, d, fill_bits=0xFFFF)
    table = [4, 1, 3]
    n = 10
    k = rng.integers(0, 2 ** 16, size=(n, H, d), dtype=np.uint16)
    v = rng.integers(0, 2 ** 16, size=(n, H, d), dtype=np.uint16)
    slots = [table[t // B] * B + t % B for t in range(n)]
    write_kv(pool, 1, k, v, slots)
    Kc, Vc = gather(pool, 1, table, n)
    assert np.array_equal(Kc, k) and np.array_equal(Vc, v)
    # layer 0 untouched; negative slots skipped
    assert np.all(pool.K[0] == 0xFFFF)
    before = pool.K.copy()
    write_kv(pool, 1, k[:2], v[:2], [-1, -5])
    assert np.array_equal(before, pool.K)
    # exact placement: token 5 -> logical block 1 (phys 1), offset 1
    assert np.array_equal(pool.K[1, 1, :, 1, :], k[5])


def test_copy_blocks_whole_block_every_layer():
    rng = np.random.default_rng(1)
    pool = HostPool(3, 5, 2, 4, 8)
    pool.K[:] = rng.integers(0, 2 ** 16, size=pool.K.shape, dtype=np.uint16)
    pool.V[:] = rng.integers(0, 2 ** 16, size=pool.V.shape, dtype=np.uint16)
    K0, V0 = pool.K.copy(), pool.V.copy()
    copy_blocks(pool, [(2, 4), (0, 1)])
    assert np.array_equal(pool.K[:, 4], K0[:, 2]) and np.array_equal(pool.V[:, 4], V0[:, 2])
    assert np.array_equal(pool.K[:, 1], K0[:, 0]) and np.array_equal(pool.V[:, 1], V0[:, 0])
    for b in (0, 2, 3):
        assert np.array_equal(pool.K[:, b], K0[:, b])


def test_physical_block_permutation_leaves_output_bitwise_unchanged():
    rng = np.random.default_rng(2)
    L, P, H, B, d, Hq = 1, 12, 2, 4, 16, 4
    pool = HostPool(L, P, H, B, d)
    pool.K[:] = round_to_dtype_bits(rng.standard_normal(pool.K.shape).astype(np.float32), "f16")
    pool.V[:] = round_to_dtype_bits(rng.standard_normal(pool.V.shape).astype(np.float32), "f16")
    tables = [[3, 7, 1], [0, 5, 9, 2]]
    lens = [10, 15]
    q = round_to_dtype_bits(rng.standard_normal((2, Hq, d)).astype(np.float32), "f16")
    ref = decode_layer(pool, 0, q, tables, lens, 0.25, "f16")
    perm = rng.permutation(P)                   # physical block b moves to perm[b]
    moved = HostPool(L, P, H, B, d)
    moved.K[:, perm] = pool.K
    moved.V[:, perm] = pool.V
    tables2 = [[int(perm[b]) for b in t] for t in tables]
    out = decode_layer(moved, 0, q, tables2, lens, 0.25, "f16")
    assert np.array_equal(ref, out)
    # and the paged result is the contiguous-baseline result
    Kc, Vc = gather(pool, 0, tables[1], lens[1])
    dense = dense_attention(bits_to_f64(q[1], "f16"), bits_to_f64(Kc, "f16"),
                            bits_to_f64(Vc, "f16"), 0.25)
    assert np.array_equal(dense, ref[1])


def test_tail_slots_and_unused_blocks_never_read():
    wl = make_workload(1)
    nan = dtype_nan_bits("f16")
    st = build_state(wl, layers=(0,), fill_bits=nan)
    out, slots, pairs = decode_step(st, wl)
    assert np.all(np.isfinite(out))
    # every position a sequence attends to holds a finite value
    for s, n in enumerate(st.lens):
        Kc, Vc = gather(st.pool, 0, st.tables[s], n)
        assert np.all(np.isfinite(f16_bits_to_f64(Kc)))


def test_config2_copy_on_write_isolates_sharers():
    wl = make_workload(2)
    st = build_state(wl, layers=(0,), fill_bits=dtype_nan_bits("f16"))
    p1 = st.tables[1][1]
    k_p1_before = st.pool.K[0, p1].copy()
    # outputs of sequences 1..3 computed without sequence 0's step
    q = wl.q_bits(0)
    lens_after = [n + 1 for n in st.lens]
    out, slots, pairs = decode_step(st, wl)
    assert len(pairs) == 1
    assert np.array_equal(st.pool.K[0, p1], k_p1_before)       # original untouched
    new = pairs[0][1]
    # the copy equals the original except the slot sequence 0 just wrote
    diff = np.any(st.pool.K[0, new] != k_p1_before, axis=(0, 2))
    assert list(np.nonzero(diff)[0]) == [36 % 32]
    # sequence 0 sees its own new token, not the sharers' token 36
    Kc, _ = gather(st.pool, 0, st.tables[0], lens_after[0])
    assert np.array_equal(Kc[36], wl.knew_bits(0)[0])
    Kc1, _ = gather(st.pool, 0, st.tables[1], lens_after[1])
    assert not np.array_equal(Kc1[36], wl.knew_bits(0)[0])
    for s in (1, 2, 3):
        assert np.array_equal(
            out[0, s], decode_one(st.pool, 0, q[s], st.tables[s], lens_after[s], float(wl.scale), "f16"))
