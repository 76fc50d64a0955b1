"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Integer and byte work (slot scatter, block copies, tables, refcounts,
copy-on-write pairs) must be bit-exact; attention must be within the stated
bounds of the oracle: every element within 2e-3 (fp16) or 2e-3 plus half an
output ulp (bf16, whose rounding alone exceeds 2e-3 above 0.5), and relative
error at most 1e-2 wherever |ref| >= 0.2."""

import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle.attention import dense_attention
from oracle.cache_ops import HostPool, copy_blocks, gather, write_kv
from oracle.decode import decode_layer
from oracle.dtypes import bits_to_f64
from oracle.replay import build_state, decode_step
from tests.harness import (OracleSide, fill_pool_nan, fill_pool_random, layer_inputs, make_engine,
                           replay_history_device, snapshot_layers, to_device_bits, to_host_bits,
                           to_host_f64, tol_stats, within_tolerance, check_prefix_groups)
from workloads import make_workload, normal_bits, round_to_dtype_bits, with_headroom
from workloads.gen import dtype_nan_bits

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _gpu_required():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _pool(L, Hkv, B, P, dtype, order=None):
    from paged_kv_cache_239_amd import Pool
    return Pool(L, Hkv, 128, B, P, dtype, free_order=order)


# --------------------------------------------------------------------------------
# write_kv and copy_blocks: bit-exact
# --------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,B,Hkv", [("f16", 16, 2), ("bf16", 32, 8), ("f16", 16, 40), ("bf16", 8, 4),
                                         ("f16", 128, 2)])
def test_write_kv_bit_exact(dtype, B, Hkv):
    _say(f"write_kv {dtype} B={B} Hkv={Hkv}")
    rng = np.random.default_rng(1)
    L, P, S = 3, 24, 37
    pool = _pool(L, Hkv, B, P, dtype)
    init = rng.integers(0, 2 ** 16, size=pool.nbytes // 2, dtype=np.uint16)
    pool.buffer.view(torch.int16).copy_(torch.from_numpy(init.view(np.int16)))
    host = HostPool.from_arrays(init.reshape(L, 2, P, Hkv, B, 128)[:, 0].copy(),
                                init.reshape(L, 2, P, Hkv, B, 128)[:, 1].copy())
    slots = rng.choice(P * B, size=S, replace=False).astype(np.int64)
    slots[[3, 10]] = -1                         # skipped tokens
    slots[5] = P * B + 7                        # beyond the pool: ignored
    k = normal_bits(rng, (S, Hkv, 128), dtype)
    v = normal_bits(rng, (S, Hkv, 128), dtype)
    layer = 1
    pool.write_kv(layer, to_device_bits(k, dtype), to_device_bits(v, dtype), torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    oslots = [int(x) if x < P * B else -1 for x in slots]
    write_kv(host, layer, k, v, oslots)
    for l in range(L):
        assert np.array_equal(to_host_bits(pool.slab(l, "k")), host.K[l])
        assert np.array_equal(to_host_bits(pool.slab(l, "v")), host.V[l])


@pytest.mark.parametrize("dtype,B,Hkv,L", [("f16", 32, 2, 1), ("f16", 16, 40, 3), ("bf16", 16, 8, 2),
                                           ("bf16", 8, 4, 2), ("f16", 128, 2, 2)])
def test_copy_blocks_bit_exact(dtype, B, Hkv, L):
    _say(f"copy_blocks {dtype} B={B} Hkv={Hkv} L={L}")
    rng = np.random.default_rng(2)
    P = 20
    pool = _pool(L, Hkv, B, P, dtype)
    init = rng.integers(0, 2 ** 16, size=pool.nbytes // 2, dtype=np.uint16)
    pool.buffer.view(torch.int16).copy_(torch.from_numpy(init.view(np.int16)))
    host = HostPool.from_arrays(init.reshape(L, 2, P, Hkv, B, 128)[:, 0].copy(),
                                init.reshape(L, 2, P, Hkv, B, 128)[:, 1].copy())
    pairs = np.array([[3, 11], [0, 19], [7, 2], [5, 5], [4, 25]], dtype=np.int32)
    pool.copy_blocks(torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    copy_blocks(host, [(3, 11), (0, 19), (7, 2)])   # src == dst and out-of-range pairs are skipped
    for l in range(L):
        assert np.array_equal(to_host_bits(pool.slab(l, "k")), host.K[l])
        assert np.array_equal(to_host_bits(pool.slab(l, "v")), host.V[l])


# --------------------------------------------------------------------------------
# decode attention on the small workloads: full step vs oracle
# --------------------------------------------------------------------------------
def _small_workload_step(cfg, steps=1, fused=True, block_size=None, grouped=False):
    wl = with_headroom(make_workload(cfg, block_size=block_size), steps)
    c = wl.cfg
    eng = make_engine(wl, steps=steps, fused=fused, grouped=grouped)
    fill_pool_nan(eng, c.dtype)                 # unwritten slots hold NaN
    replay_history_device(eng, wl, write_values=True)
    st = build_state(wl, layers=tuple(range(c.L)), maxb=wl.max_blocks(steps), fill_bits=dtype_nan_bits(c.dtype))
    results = []
    for step in range(steps):
        qs, ks, vs = layer_inputs(wl, range(c.L), step)
        outs = {l: torch.empty_like(qs[l]) for l in range(c.L)}
        max_ctx = eng.manager_step()
        eng.device_step(qs, ks, vs, outs, max_ctx, float(wl.scale))
        torch.cuda.synchronize()
        ref, slots, pairs = decode_step(st, wl, step)
        assert list(eng.last_slots) == slots
        assert [tuple(p) for p in eng.last_pairs.tolist()] == pairs
        got = np.stack([to_host_f64(outs[l], c.dtype) for l in range(c.L)])
        results.append((got, ref, pairs))
    return wl, eng, st, results


@pytest.mark.parametrize("fused", [True, False])
def test_config1_five_lengths_gqa4_b16(fused):
    _say(f"config 1 fused={fused}")
    wl, eng, st, res = _small_workload_step(1, fused=fused)
    got, ref, pairs = res[0]
    ok, stats = within_tolerance(got, ref, wl.cfg.dtype)
    _say(f"config 1 stats {stats}")
    assert ok, stats
    assert pairs == []
    # paged tables as the worked example: 62 blocks, the first 62 of the permutation
    assert eng.pool.stats()["allocs"] == 62


@pytest.mark.parametrize("fused", [True, False])
def test_config2_prefix_sharing_cow(fused):
    _say(f"config 2 fused={fused}")
    wl, eng, st, res = _small_workload_step(2, steps=2, fused=fused)
    for got, ref, pairs in res:
        ok, stats = within_tolerance(got, ref, wl.cfg.dtype)
        _say(f"config 2 stats {stats}")
        assert ok, stats
    assert len(res[0][2]) == 1 and res[1][2] == []
    # device pool equals the oracle pool byte for byte (copy + writes), both layers' K and V
    assert np.array_equal(to_host_bits(eng.pool.slab(0, "k")), st.pool.K[0])
    assert np.array_equal(to_host_bits(eng.pool.slab(0, "v")), st.pool.V[0])
    # refcounts and free list match
    assert eng.pool.refcounts() == st.mgr.ref
    assert eng.pool.free_list() == st.mgr.free_list()


def test_config2_isolation_sharers_unchanged():
    """Sequences 2-4 produce the same output whether or not sequence 1's
    copy-on-write write happened in the same step."""
    _say("config 2 isolation")
    wl = make_workload(2)
    c = wl.cfg
    eng = make_engine(wl)
    fill_pool_nan(eng, c.dtype)
    replay_history_device(eng, wl, write_values=True)
    p1 = int(eng.tables[1][1])
    before = to_host_bits(eng.pool.slab(0, "k"))[p1].copy()
    qs, ks, vs = layer_inputs(wl, [0], 0)
    out = {0: torch.empty_like(qs[0])}
    max_ctx = eng.manager_step()
    eng.device_step(qs, ks, vs, out, max_ctx, float(wl.scale))
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(eng.pool.slab(0, "k"))[p1], before)
    got = to_host_f64(out[0], c.dtype)
    # recompute sharers alone (the oracle without sequence 0's step)
    st = build_state(wl, layers=(0,), fill_bits=dtype_nan_bits(c.dtype))
    lens = [n + 1 for n in st.lens]
    from oracle.manager import BlockManager
    for s in (1, 2, 3):
        t = list(st.tables[s])
        st.mgr.append_slot(t, st.lens[s])
        slot = t[(lens[s] - 1) // c.B] * c.B + (lens[s] - 1) % c.B
        write_kv(st.pool, 0, wl.knew_bits(0)[s:s + 1], wl.vnew_bits(0)[s:s + 1], [slot])
        ref = decode_layer(st.pool, 0, wl.q_bits(0)[s:s + 1], [t], [lens[s]], float(wl.scale), c.dtype)[0]
        ok, stats = within_tolerance(got[s], ref, c.dtype)
        assert ok, (s, stats)


# --------------------------------------------------------------------------------
# decode attention over shapes, lengths and dtypes
# --------------------------------------------------------------------------------
def _direct_case(rng, S, Hq, Hkv, B, dtype, lens, P=None, poison=True, q_scale=1.0, order=None):
    """Pool filled with random values (NaN outside live slots), random tables."""
    maxb = max(1, max(-(-n // B) for n in lens))
    need = sum(-(-n // B) for n in lens)
    P = P or need + 3
    pool = _pool(1, Hkv, B, P, dtype, order)
    shape = (1, P, Hkv, B, 128)
    K = normal_bits(rng, shape, dtype)
    V = normal_bits(rng, shape, dtype)
    perm = rng.permutation(P)
    tables = np.full((S, maxb), -1, dtype=np.int32)
    o = 0
    live = np.zeros((P, B), dtype=bool)
    for s, n in enumerate(lens):
        nb = -(-n // B)
        tables[s, :nb] = perm[o:o + nb]
        o += nb
        for t in range(n):
            live[tables[s, t // B], t % B] = True
    if poison:
        nan = dtype_nan_bits(dtype)
        dead = np.broadcast_to(~live[:, None, :], (P, Hkv, B))
        K[0][dead] = nan
        V[0][dead] = nan
        tables[tables < 0] = 10 ** 6            # padding entries: out of range, never read
    pool.slab(0, "k").view(torch.int16).copy_(torch.from_numpy(K[0].view(np.int16)))
    pool.slab(0, "v").view(torch.int16).copy_(torch.from_numpy(V[0].view(np.int16)))
    q = round_to_dtype_bits(rng.standard_normal((S, Hq, 128)).astype(np.float32) * q_scale, dtype)
    host = HostPool.from_arrays(K, V)
    return pool, host, tables, q


def _run_direct(pool, tables, q, lens, dtype, scale, max_ctx=None):
    from paged_kv_cache_239_amd import decode_workspace
    S, Hq = q.shape[0], q.shape[1]
    max_ctx = max(lens) if max_ctx is None else max_ctx
    ws = decode_workspace(pool, S, Hq, max_ctx)
    dq = to_device_bits(q, dtype)
    out = torch.empty_like(dq)
    pool.decode_attention(0, out, dq, torch.from_numpy(tables).cuda(),
                          torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda(), max_ctx, scale, workspace=ws)
    torch.cuda.synchronize()
    return out


SHAPES = [
    # (G, Hkv, B, dtype)
    (1, 4, 16, "f16"), (2, 2, 16, "bf16"), (4, 2, 16, "f16"), (8, 1, 16, "bf16"),
    (1, 2, 32, "bf16"), (2, 4, 32, "f16"), (4, 8, 32, "bf16"), (8, 2, 32, "f16"),
    (1, 4, 8, "f16"), (4, 2, 8, "bf16"), (8, 1, 8, "f16"),
    (2, 2, 64, "bf16"), (4, 8, 64, "f16"),
    (1, 2, 128, "bf16"), (4, 2, 128, "f16"), (8, 2, 128, "bf16"),
]


@pytest.mark.parametrize("G,Hkv,B,dtype", SHAPES)
def test_decode_shapes_ragged_lengths(G, Hkv, B, dtype):
    _say(f"shape G={G} Hkv={Hkv} B={B} {dtype}")
    rng = np.random.default_rng(10 * G + B)
    lens = [1, 2, 15, 16, 17, 31, 33, 64, 100, 257, 511, 1000, 1537, 2048, 3001]
    if B == 32:
        lens = lens + [32, 63, 4096]
    lens = lens + [B - 1, B, B + 1, 2 * B + 3]   # around this block size's boundaries
    S = len(lens)
    Hq = G * Hkv
    pool, host, tables, q = _direct_case(rng, S, Hq, Hkv, B, dtype, lens)
    scale = float(np.float32(1 / np.sqrt(128)))
    out = _run_direct(pool, tables, q, lens, dtype, scale)
    got = to_host_f64(out, dtype)
    ref = decode_layer(host, 0, q, tables, lens, scale, dtype)
    ok, stats = within_tolerance(got, ref, dtype)
    _say(f"stats {stats}")
    assert ok, stats


def test_decode_zero_length_gives_zero_and_single_token_gives_value():
    _say("edge lengths")
    rng = np.random.default_rng(3)
    lens = [0, 1, 0, 5]
    pool, host, tables, q = _direct_case(rng, 4, 8, 2, 16, "f16", [max(n, 1) for n in lens])
    out = _run_direct(pool, tables, q, lens, "f16", 0.1)
    got = to_host_f64(out, "f16")
    assert np.all(got[0] == 0) and np.all(got[2] == 0)
    # one token: output is that token's value, exactly (rounded back to fp16)
    v0 = bits_to_f64(host.V[0, tables[1, 0], :, 0, :], "f16")       # [Hkv][d]
    assert np.array_equal(got[1], np.repeat(v0, 4, axis=0))
    ref = decode_layer(host, 0, q[3:4], tables[3:4], [5], 0.1, "f16")
    assert within_tolerance(got[3], ref[0], "f16")[0]


@pytest.mark.parametrize("mag", [30.0, 300.0])
def test_decode_extreme_logits(mag):
    """Scores of order +-1e3 .. 1e4 must neither overflow nor lose the maximum."""
    _say(f"extreme logits {mag}")
    rng = np.random.default_rng(4)
    lens = [700, 2000, 64]
    pool, host, tables, q = _direct_case(rng, 3, 8, 2, 16, "f16", lens, q_scale=mag)
    scale = 1.0
    out = _run_direct(pool, tables, q, lens, "f16", scale)
    got = to_host_f64(out, "f16")
    ref = decode_layer(host, 0, q, tables, lens, scale, "f16")
    assert np.all(np.isfinite(got))
    ok, st = within_tolerance(got, ref, "f16")
    _say(f"stats {st}")
    assert ok and st["allclose_worst"] <= 0, st


def test_decode_bitwise_invariant_under_block_permutation_and_reruns():
    _say("permutation invariance")
    rng = np.random.default_rng(5)
    lens = [300, 1234, 77, 2500]
    dtype = "bf16"
    pool, host, tables, q = _direct_case(rng, 4, 16, 4, 16, dtype, lens, poison=False)
    scale = 0.0883883
    out1 = _run_direct(pool, tables, q, lens, dtype, scale)
    out2 = _run_direct(pool, tables, q, lens, dtype, scale)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    # move every physical block b to perm[b] and rewrite the tables
    P = host.P
    perm = rng.permutation(P)
    K2 = np.empty_like(host.K)
    V2 = np.empty_like(host.V)
    K2[:, perm] = host.K
    V2[:, perm] = host.V
    pool.slab(0, "k").view(torch.int16).copy_(torch.from_numpy(K2[0].view(np.int16)))
    pool.slab(0, "v").view(torch.int16).copy_(torch.from_numpy(V2[0].view(np.int16)))
    t2 = np.where(tables >= 0, perm[np.clip(tables, 0, P - 1)], tables).astype(np.int32)
    out3 = _run_direct(pool, t2, q, lens, dtype, scale)
    assert torch.equal(out1.view(torch.int16), out3.view(torch.int16))


def test_decode_partition_merge_with_garbage_and_reused_workspace():
    """Every partial the merge reads is written by the same call: a
    workspace full of garbage (all-ones bytes, which are NaN partials, then
    random bytes) and a workspace reused by the previous call must both give
    the oracle's result.  One context of 30,000 tokens spreads over 79
    partitions."""
    _say("partition merge: garbage and reused workspace")
    rng = np.random.default_rng(7)
    lens = [30000, 777, 5000, 1, 1600, 384, 385, 12345]
    dtype = "f16"
    Hkv, G = 2, 4
    pool, host, tables, q = _direct_case(rng, len(lens), G * Hkv, Hkv, 16, dtype, lens)
    scale = float(np.float32(1 / np.sqrt(128)))
    S, Hq = q.shape[0], q.shape[1]
    max_ctx = max(lens)
    nbytes = pool.workspace_bytes(S, Hq, max_ctx)
    assert nbytes > 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    d_tables = torch.from_numpy(tables).cuda()
    d_lens = torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda()
    ref = decode_layer(host, 0, q, tables, lens, scale, dtype)
    q2 = round_to_dtype_bits(rng.standard_normal(q.shape).astype(np.float32), dtype)
    ref2 = decode_layer(host, 0, q2, tables, lens, scale, dtype)
    fills = [("all-ones bytes", lambda: ws.fill_(255)),
             ("random bytes", lambda: ws.copy_(torch.from_numpy(rng.integers(0, 256, nbytes, dtype=np.uint8)))),
             ("reused", lambda: None)]
    for (name, fill), (qq, rr) in zip(fills, [(q, ref), (q2, ref2), (q, ref)]):
        fill()
        dq = to_device_bits(qq, dtype)
        out = torch.empty_like(dq)
        pool.decode_attention(0, out, dq, d_tables, d_lens, max_ctx, scale, workspace=ws)
        torch.cuda.synchronize()
        ok, stats = within_tolerance(to_host_f64(out, dtype), rr, dtype)
        _say(f"{name}: {stats}")
        assert ok, (name, stats)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("case,G,B,dtype", [("ragged", 4, 16, "bf16"), ("many", 4, 16, "bf16"),
                                            ("ragged", 1, 8, "f16"), ("ragged", 2, 32, "bf16"),
                                            ("ragged", 8, 128, "f16")])
def test_decode_ordered_matches_oracle_and_fixed_order(fused, case, G, B, dtype):
    """Partitions of equal length launched longest first from host copies
    of the lengths: the oracle's outputs within tolerance, the same bits on
    a rerun, and (fused) the same pool as the fixed grid order; empty
    sequences, lengths at and around partition multiples.  "many" has more
    (sequence, partition) units than one list holds and runs as the fixed
    order does, bit for bit."""
    _say(f"ordered launch {case} G={G} B={B} {dtype} fused={fused}")
    rng = np.random.default_rng(11 + G + B)
    Hkv = 2
    if case == "ragged":
        lens = [0, 1, 383, 384, 385, 767, 768, 769, 1536, 2047, 4096, 5000, 12345, 3, 0, 900]
    else:
        lens = [int(x) for x in rng.integers(1, 100, size=600)]
    S, Hq = len(lens), G * Hkv
    pool, host, tables, q = _direct_case(rng, S, Hq, Hkv, B, dtype, [max(n, 1) for n in lens])
    scale = float(np.float32(1 / np.sqrt(128)))
    max_ctx = max(lens)
    from paged_kv_cache_239_amd import decode_workspace
    ws = decode_workspace(pool, S, Hq, max_ctx)
    d_tables = torch.from_numpy(tables).cuda()
    hl = np.asarray(lens, dtype=np.int32)
    d_lens = torch.from_numpy(hl).cuda()
    dq = to_device_bits(q, dtype)
    knew = normal_bits(rng, (S, Hkv, 128), dtype)
    vnew = normal_bits(rng, (S, Hkv, 128), dtype)
    slots = np.array([int(tables[s, (n - 1) // B]) * B + (n - 1) % B if n > 0 else -1
                      for s, n in enumerate(lens)], dtype=np.int64)
    dk, dv, ds = to_device_bits(knew, dtype), to_device_bits(vnew, dtype), torch.from_numpy(slots).cuda()
    out_fixed, out_ord = torch.empty_like(dq), torch.empty_like(dq)
    if fused:
        pool.write_kv_decode_attention(0, dk, dv, ds, out_fixed, dq, d_tables, d_lens, max_ctx, scale, workspace=ws)
        torch.cuda.synchronize()
        pool_fixed = to_host_bits(pool.buffer).copy()
        pool.decode_attention_ordered(0, out_ord, dq, d_tables, d_lens, hl, max_ctx, scale, workspace=ws,
                                      k=dk, v=dv, slot_mapping=ds)
        torch.cuda.synchronize()
        assert np.array_equal(to_host_bits(pool.buffer), pool_fixed)
        write_kv(host, 0, knew, vnew, [int(x) for x in slots])
    else:
        pool.decode_attention(0, out_fixed, dq, d_tables, d_lens, max_ctx, scale, workspace=ws)
        pool.decode_attention_ordered(0, out_ord, dq, d_tables, d_lens, hl, max_ctx, scale, workspace=ws)
        torch.cuda.synchronize()
    again = torch.empty_like(dq)
    pool.decode_attention_ordered(0, again, dq, d_tables, d_lens, hl, max_ctx, scale, workspace=ws,
                                  k=dk if fused else None, v=dv if fused else None,
                                  slot_mapping=ds if fused else None)
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.int16), out_ord.view(torch.int16))
    if case == "many":
        assert torch.equal(out_fixed.view(torch.int16), out_ord.view(torch.int16))
    for o in (out_fixed, out_ord):
        assert within_tolerance(to_host_f64(o, dtype)[[s for s, n in enumerate(lens) if n > 0]],
                                decode_layer(host, 0, q[[s for s, n in enumerate(lens) if n > 0]],
                                             tables[[s for s, n in enumerate(lens) if n > 0]],
                                             [n for n in lens if n > 0], scale, dtype), dtype)[0]
    got = to_host_f64(out_ord, dtype)
    live = [s for s, n in enumerate(lens) if n > 0]
    assert np.all(got[[s for s, n in enumerate(lens) if n == 0]] == 0)
    ref = decode_layer(host, 0, q[live], tables[live], [lens[s] for s in live], scale, dtype)
    ok, stats = within_tolerance(got[live], ref, dtype)
    _say(f"stats {stats}")
    assert ok, stats


def test_decode_ordered_rejects_partial_fused_arguments():
    rng = np.random.default_rng(12)
    pool, host, tables, q = _direct_case(rng, 2, 4, 2, 16, "f16", [10, 20])
    from paged_kv_cache_239_amd import PAError
    dq = to_device_bits(q, "f16")
    out = torch.empty_like(dq)
    d_tables = torch.from_numpy(tables).cuda()
    d_lens = torch.tensor([10, 20], dtype=torch.int32, device="cuda")
    k = torch.zeros((2, 2, 128), dtype=torch.float16, device="cuda")
    with pytest.raises(PAError):
        pool.decode_attention_ordered(0, out, dq, d_tables, d_lens, np.array([10, 20], np.int32), 20, 0.1, k=k)


def test_decode_matches_contiguous_baseline():
    """Paged result vs the oracle's dense attention on contiguous K/V."""
    _say("contiguous baseline")
    rng = np.random.default_rng(6)
    lens = [513, 100]
    pool, host, tables, q = _direct_case(rng, 2, 4, 1, 16, "f16", lens)
    out = _run_direct(pool, tables, q, lens, "f16", 0.125)
    got = to_host_f64(out, "f16")
    for s, n in enumerate(lens):
        Kc, Vc = gather(host, 0, tables[s], n)
        dense = dense_attention(bits_to_f64(q[s], "f16"), bits_to_f64(Kc, "f16"), bits_to_f64(Vc, "f16"), 0.125)
        assert within_tolerance(got[s], dense, "f16")[0]


# --------------------------------------------------------------------------------
# full-size workloads: sampled outputs, in the bench's launch configuration
# --------------------------------------------------------------------------------
def _full_size(cfg, steps, layers, seqs_per_layer, seed, fused=True, block_size=None, grouped=False,
               head_shards=1):
    wl = with_headroom(make_workload(cfg, block_size=block_size, head_shards=head_shards), steps)
    c = wl.cfg
    eng = make_engine(wl, steps=steps, fused=fused, grouped=grouped)
    _say(f"config {cfg}: pool {eng.pool.nbytes / 2**30:.1f} GiB, P={wl.P}, S={wl.S}")
    fill_pool_random(eng, wl)
    replay_history_device(eng, wl, write_values=False)
    snaps = snapshot_layers(eng, layers)
    ora = OracleSide(wl, snaps, wl.max_blocks(steps))
    assert list(eng.lens) == ora.state.lens
    rng = np.random.default_rng(seed)
    worst = {}
    for step in range(steps):
        qs, ks, vs = layer_inputs(wl, range(c.L), step)
        outs = {l: torch.empty_like(qs[l]) for l in range(c.L)}
        if c.beam:
            eng.reorder(wl.parents(step))
        max_ctx = eng.manager_step()
        eng.device_step(qs, ks, vs, outs, max_ctx, float(wl.scale))
        torch.cuda.synchronize()
        slots, pairs, lens = ora.step(step)
        assert list(eng.last_slots) == slots
        assert [tuple(p) for p in eng.last_pairs.tolist()] == pairs
        assert list(eng.lens) == lens
        for layer in layers:
            got_all = to_host_f64(outs[layer], c.dtype)
            pick = rng.choice(wl.S, size=min(seqs_per_layer, wl.S), replace=False)
            pick = sorted(set(pick.tolist()) | {int(np.argmax(lens)), int(np.argmin(lens))})
            for s in pick:
                ref = ora.expected(layer, s, step)
                ok, stats = within_tolerance(got_all[s], ref, c.dtype)
                assert ok, (cfg, step, layer, s, stats)
                worst[(step, layer, s)] = stats["max_abs"]
        _say(f"config {cfg} step {step}: pairs={len(pairs)} worst max_abs {max(worst.values()):.2e}")
    # the oracle-side pools saw the same copies and writes: compare sampled layers byte for byte
    for layer in layers:
        assert np.array_equal(to_host_bits(eng.pool.slab(layer, "k")), ora.pools[layer].K[0])
        assert np.array_equal(to_host_bits(eng.pool.slab(layer, "v")), ora.pools[layer].V[0])
    assert eng.pool.refcounts() == ora.state.mgr.ref
    del eng
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fused", [True, False])
def test_config3_full_size_sampled(fused):
    _full_size(3, steps=2, layers=[0, 31], seqs_per_layer=6, seed=30, fused=fused)


def test_config4_full_size_sampled():
    _full_size(4, steps=1, layers=[0, 17], seqs_per_layer=3, seed=40)


def test_config5_full_size_sampled():
    _full_size(5, steps=2, layers=[0, 39], seqs_per_layer=6, seed=50)


def test_config6_beam_search_sampled():
    """Beam reselection before every step: forks, frees, copy-on-write of
    shared last blocks, then the fused write and attention."""
    _full_size(6, steps=4, layers=[0, 39], seqs_per_layer=8, seed=66)


@pytest.mark.parametrize("B", [8, 32, 64, 128])
def test_config3_other_block_sizes_sampled(B):
    """The config-3 batch stored in blocks of B tokens (block-size sweep)."""
    _full_size(3, steps=2, layers=[0, 31], seqs_per_layer=4, seed=60 + B, block_size=B)


@pytest.mark.parametrize("shards", [2, 8])
def test_config3_head_shard_sampled(shards):
    """One GPU's share of the config-3 heads when they are split over
    `shards` GPUs (8 shards: 4 query heads over 1 key/value head): a smaller
    grid, so shorter partitions and more of them per sequence."""
    _full_size(3, steps=2, layers=[0, 31], seqs_per_layer=6, seed=70 + shards, head_shards=shards)


@pytest.mark.parametrize("cfg", [1, 2])
def test_small_workloads_at_every_block_size(cfg):
    """Each block size: full parity with the oracle over two fused steps, the
    oracle's slots and copies, and outputs bitwise equal to every other block
    size (the kernel's accumulation order depends on 16-token steps and
    partitions only, never on where blocks start)."""
    base = None
    for B in (8, 16, 32, 64, 128):
        _say(f"config {cfg} at B={B}")
        wl, eng, st, results = _small_workload_step(cfg, steps=2, fused=True, block_size=B)
        outs = []
        for got, ref, pairs in results:
            ok, stats = within_tolerance(got, ref, wl.cfg.dtype)
            assert ok, (B, stats)
            outs.append(got)
        outs = np.stack(outs)
        if base is None:
            base = outs
        else:
            assert np.array_equal(outs, base), B
        del eng


@pytest.mark.parametrize("cfg,steps,grouped", [(1, 2, False), (2, 2, False), (5, 1, False), (6, 2, False),
                                               (5, 1, True), (6, 2, True)])
def test_fused_write_attention_equals_separate_calls(cfg, steps, grouped):
    """pa_write_kv_decode_attention == pa_write_kv then pa_decode_attention
    (grouped: pa_decode_attention_grouped with and without the cache write):
    outputs and the whole pool byte for byte."""
    _say(f"fused vs separate, config {cfg} grouped={grouped}")
    wl = make_workload(cfg)
    c = wl.cfg
    engines = []
    for fused in (True, False):
        eng = make_engine(wl, steps=steps, fused=fused, grouped=grouped)
        if cfg in (5, 6):
            fill_pool_random(eng, wl)
            replay_history_device(eng, wl, write_values=False)
        else:
            fill_pool_nan(eng, c.dtype)
            replay_history_device(eng, wl, write_values=True)
        engines.append(eng)
    for step in range(steps):
        qs, ks, vs = layer_inputs(wl, range(c.L), step)
        outs = []
        for eng in engines:
            o = {l: torch.empty_like(qs[l]) for l in range(c.L)}
            if c.beam:
                eng.reorder(wl.parents(step))
            max_ctx = eng.manager_step()
            eng.device_step(qs, ks, vs, o, max_ctx, float(wl.scale))
            outs.append(o)
        torch.cuda.synchronize()
        for l in range(c.L):
            assert torch.equal(outs[0][l].view(torch.int16), outs[1][l].view(torch.int16)), (cfg, step, l)
    assert torch.equal(engines[0].pool.buffer, engines[1].pool.buffer)


# --------------------------------------------------------------------------------
# swap-out / swap-in through pinned host memory
# --------------------------------------------------------------------------------
@pytest.mark.parametrize("B,dtype", [(8, "bf16"), (16, "f16"), (128, "bf16")])
def test_swap_round_trip_through_host_pool(B, dtype):
    """A group of sequences sharing a prefix moves to a pinned host pool and
    back (pa_move_blocks + pa_swap_blocks): the host pool's bytes equal the
    oracle's copy, the device blocks come back bit for bit although the
    freed originals were overwritten meanwhile, and attention over the group
    is bitwise unchanged."""
    from oracle.manager import BlockManager
    from oracle.swap import copy_between, move_blocks
    from paged_kv_cache_239_amd import Pool, decode_workspace
    _say(f"swap B={B} {dtype}")
    rng = np.random.default_rng(77 + B)
    L, Hkv, Hq, P, Pc = 2, 4, 8, 96, 64
    order, corder = rng.permutation(P).astype(np.int32), rng.permutation(Pc).astype(np.int32)
    dev = Pool(L, Hkv, 128, B, P, dtype, free_order=order)
    host = Pool(L, Hkv, 128, B, Pc, dtype, free_order=corder, device="pinned")
    init = rng.integers(0, 2 ** 16, size=dev.nbytes // 2, dtype=np.uint16) & 0xBFFF   # finite values
    dev.buffer.view(torch.int16).copy_(torch.from_numpy(init.view(np.int16)))
    ora_dev, ora_host = BlockManager(P, B, order), BlockManager(Pc, B, corder)
    hp_dev = HostPool.from_arrays(init.reshape(L, 2, P, Hkv, B, 128)[:, 0].copy(),
                                  init.reshape(L, 2, P, Hkv, B, 128)[:, 1].copy())
    hp_host = HostPool(L, Pc, Hkv, B, 128)
    # a prompt of 3.5 blocks, three beams forked from it with own tails; one other sequence
    maxb = 16
    n_prompt = 3 * B + B // 2
    tables = np.full((4, maxb), -1, dtype=np.int32)
    o_tables = [[-1] * maxb for _ in range(4)]
    root = np.full(maxb, -1, dtype=np.int32)
    o_root = [-1] * maxb
    dev.append_tokens(root, 0, n_prompt)
    ora_dev.append_tokens(o_root, 0, n_prompt)
    lens = [n_prompt + 5, n_prompt + B + 1, n_prompt + 2, 2 * B + 3]
    for s in range(3):
        dev.fork(root, n_prompt, tables[s])
        o_tables[s][: -(-n_prompt // B)] = ora_dev.fork(o_root, n_prompt)
        _, pairs = dev.append_tokens(tables[s], n_prompt, lens[s] - n_prompt)
        _, o_pairs = ora_dev.append_tokens(o_tables[s], n_prompt, lens[s] - n_prompt)
        assert [tuple(p) for p in pairs] == o_pairs
        if pairs:
            dev.copy_blocks(torch.tensor(pairs, dtype=torch.int32, device="cuda"))
            copy_blocks(hp_dev, o_pairs)
    dev.free_seq(root, n_prompt)
    ora_dev.free_seq(o_root, n_prompt)
    dev.append_tokens(tables[3], 0, lens[3])
    ora_dev.append_tokens(o_tables[3], 0, lens[3])
    torch.cuda.synchronize()
    scale = float(np.float32(1 / np.sqrt(128)))
    q = round_to_dtype_bits(rng.standard_normal((4, Hq, 128)).astype(np.float32), dtype)
    dq = to_device_bits(q, dtype)

    def attend():
        ws = decode_workspace(dev, 4, Hq, maxb * B)
        outs = []
        for layer in range(L):
            out = torch.empty_like(dq)
            dev.decode_attention(layer, out, dq, torch.from_numpy(tables).cuda(),
                                 torch.tensor(lens, dtype=torch.int32, device="cuda"), max(lens), scale, workspace=ws)
            outs.append(out)
        torch.cuda.synchronize()
        return outs

    before = attend()
    group = tables[:3].copy()
    o_group = [list(t) for t in o_tables[:3]]
    pairs = dev.move_blocks(host, group, lens[:3])
    o_pairs = move_blocks(ora_dev, ora_host, o_group, lens[:3])
    assert [tuple(p) for p in pairs.tolist()] == o_pairs
    dev.swap_blocks(host, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    copy_between(hp_dev, hp_host, o_pairs)
    hbits = host.buffer.view(torch.int16).numpy().view(np.uint16).reshape(L, 2, Pc, Hkv, B, 128)
    assert np.array_equal(hbits[:, 0], hp_host.K) and np.array_equal(hbits[:, 1], hp_host.V)
    # the freed device blocks are reused by someone else: overwrite them
    for old, _ in o_pairs:
        for layer in range(L):
            dev.slab(layer, "k")[old].fill_(0)
            dev.slab(layer, "v")[old].fill_(0)
    back = host.move_blocks(dev, group, lens[:3])
    o_back = move_blocks(ora_host, ora_dev, o_group, lens[:3])
    assert [tuple(p) for p in back.tolist()] == o_back
    assert dev.refcounts() == ora_dev.ref and host.refcounts() == ora_host.ref
    assert dev.free_list() == ora_dev.free_list() and host.free_list() == ora_host.free_list()
    host.swap_blocks(dev, torch.from_numpy(back).cuda())
    torch.cuda.synchronize()
    tables[:3] = group
    after = attend()
    for a, b in zip(before, after):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # every block of the group holds its original bytes again
    copy_between(hp_host, hp_dev, o_back)
    for layer in range(L):
        for old_new in o_back:
            blk = old_new[1]
            assert np.array_equal(to_host_bits(dev.slab(layer, "k")[blk]), hp_dev.K[layer, blk])
            assert np.array_equal(to_host_bits(dev.slab(layer, "v")[blk]), hp_dev.V[layer, blk])


def test_swap_rejects_memory_the_device_cannot_reach():
    """A pool over ordinary (unpinned) host memory: pa_swap_blocks refuses
    before launching anything.  (The pair names blocks outside both pools, so
    even a launch would copy nothing.)"""
    from paged_kv_cache_239_amd import Pool, _abi
    dev = Pool(1, 2, 128, 16, 8, "f16")
    plain = Pool(1, 2, 128, 16, 8, "f16", device="cpu")
    pairs = torch.tensor([[100, 100]], dtype=torch.int32, device="cuda")
    with pytest.raises(_abi.PAError) as e:
        dev.swap_blocks(plain, pairs)
    assert e.value.status == _abi.PA_ERR_INVALID_ARG
    torch.cuda.synchronize()


# --------------------------------------------------------------------------------
# several queries per sequence (chunked prefill, speculative verification)
# --------------------------------------------------------------------------------
MQ_SHAPES = [
    # (G, Hkv, B, dtype)
    (1, 4, 16, "f16"), (2, 2, 32, "bf16"), (4, 2, 16, "bf16"), (8, 1, 16, "f16"),
    (4, 8, 8, "f16"), (1, 2, 128, "bf16"), (4, 2, 64, "bf16"),
]


def _mq_case(rng, G, Hkv, B, dtype, lens, nqs, ordered=False):
    from oracle.decode import multi_query_one
    from paged_kv_cache_239_amd import multi_query_workspace
    S = len(lens)
    Hq = G * Hkv
    pool, host, tables, _ = _direct_case(rng, S, Hq, Hkv, B, dtype, lens)
    T = int(sum(nqs))
    q = round_to_dtype_bits(rng.standard_normal((T, Hq, 128)).astype(np.float32), dtype)
    q_start = np.concatenate([[0], np.cumsum(nqs)]).astype(np.int32)
    scale = float(np.float32(1 / np.sqrt(128)))
    max_q = int(max(nqs))
    ws = multi_query_workspace(pool, S, Hq, max(lens), max_q)
    dq = to_device_bits(q, dtype)
    out = torch.full_like(dq, float("nan"))
    pool.multi_query_attention(0, out, dq, torch.from_numpy(q_start).cuda(), torch.from_numpy(tables).cuda(),
                               torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda(), max(lens), max_q, scale,
                               workspace=ws, host_context_lens=np.asarray(lens, dtype=np.int32) if ordered else None)
    torch.cuda.synchronize()
    got = to_host_f64(out, dtype)
    worst = 0.0
    for s in range(S):
        rows = slice(q_start[s], q_start[s + 1])
        ref = multi_query_one(host, 0, q[rows], tables[s], lens[s], scale, dtype)
        ok, st = within_tolerance(got[rows], ref, dtype)
        assert ok, (s, lens[s], nqs[s], st)
        worst = max(worst, st["max_abs"])
    return worst


@pytest.mark.parametrize("G,Hkv,B,dtype", MQ_SHAPES)
def test_multi_query_shapes_ragged(G, Hkv, B, dtype):
    _say(f"multi-query G={G} Hkv={Hkv} B={B} {dtype}")
    rng = np.random.default_rng(300 + 10 * G + B)
    lens = [1, 9, 17, 64, 100, 257, 700, 1537, 2100, 3001]
    nqs = [1, 9, 3, 64, 17, 1, 33, 8, 100, 2]        # whole prefills (nq = n), chunks and short drafts
    worst = _mq_case(rng, G, Hkv, B, dtype, lens, nqs)
    _say(f"worst max_abs {worst:.2e}")


@pytest.mark.parametrize("G,Hkv,B,dtype,max_q", [
    (4, 2, 16, "bf16", 64),      # 256 rows per sequence: four 16-row tiles per wave
    (4, 2, 8, "f16", 100),       # more rows than one workgroup holds: two row tiles
    (1, 3, 32, "bf16", 100),     # two 16-row tiles per wave
    (2, 2, 16, "f16", 20),       # one tile per wave
    (8, 1, 64, "bf16", 40),      # two workgroup row tiles of 32 query tokens
])
def test_multi_query_wide_path_both_orders(G, Hkv, B, dtype, max_q):
    """More than 32 rows per sequence: one workgroup walks a sequence's whole
    context for up to 256 rows.  Launched in the fixed order and longest
    first (host lengths); both equal the oracle within tolerance and each
    other bit for bit.  Ragged query counts up to whole prefills (nq = n),
    contexts from 1 to 3,000 positions."""
    from oracle.decode import multi_query_one
    from paged_kv_cache_239_amd import multi_query_workspace
    _say(f"multi-query wide G={G} Hkv={Hkv} B={B} {dtype} max_q={max_q}")
    rng = np.random.default_rng(7000 + 31 * G + B + max_q)
    lens = [max_q, 3000, 45, max_q + 1, 777, 2049, 130, 1, 64, 1500]
    nqs = [min(x, max_q) for x in (max_q, max_q, 45, max_q, 33, max_q - 1, 17, 1, 64, max_q)]
    S = len(lens)
    Hq = G * Hkv
    pool, host, tables, _ = _direct_case(rng, S, Hq, Hkv, B, dtype, lens)
    T = int(sum(nqs))
    q = round_to_dtype_bits(rng.standard_normal((T, Hq, 128)).astype(np.float32), dtype)
    q_start = np.concatenate([[0], np.cumsum(nqs)]).astype(np.int32)
    scale = float(np.float32(1 / np.sqrt(128)))
    ws = multi_query_workspace(pool, S, Hq, max(lens), max_q)
    dq = to_device_bits(q, dtype)
    outs = []
    for ordered in (False, True):
        out = torch.full_like(dq, float("nan"))
        pool.multi_query_attention(0, out, dq, torch.from_numpy(q_start).cuda(), torch.from_numpy(tables).cuda(),
                                   torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda(), max(lens), max_q, scale,
                                   workspace=ws, host_context_lens=np.asarray(lens, dtype=np.int32) if ordered else None)
        torch.cuda.synchronize()
        outs.append(out)
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    got = to_host_f64(outs[1], dtype)
    worst = 0.0
    for s in range(S):
        rows = slice(q_start[s], q_start[s + 1])
        ref = multi_query_one(host, 0, q[rows], tables[s], lens[s], scale, dtype)
        ok, st = within_tolerance(got[rows], ref, dtype)
        assert ok, (s, lens[s], nqs[s], st)
        worst = max(worst, st["max_abs"])
    _say(f"worst max_abs {worst:.2e}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("scale", [-0.0883883, 0.0, 0.3535534])
def test_multi_query_wide_path_scales(dtype, scale):
    """The wide path's scores enter the exponent as one fused multiply-add
    with a positive factor: a negative scale flips the query's sign, a zero
    scale gives uniform weights over the visible positions, a large one
    sharp weights.  Each against the oracle, whose softmax takes the scale
    as given."""
    from oracle.decode import multi_query_one
    from paged_kv_cache_239_amd import multi_query_workspace
    G, Hkv, B, max_q = 4, 2, 16, 64
    _say(f"multi-query wide scale={scale} {dtype}")
    rng = np.random.default_rng(7100 + int(1000 * abs(scale)) + (scale < 0))
    lens = [64, 900, 100, 333, 64 + 31]
    nqs = [64, 64, 40, 64, 64]
    S = len(lens)
    Hq = G * Hkv
    pool, host, tables, _ = _direct_case(rng, S, Hq, Hkv, B, dtype, lens)
    T = int(sum(nqs))
    q = round_to_dtype_bits(rng.standard_normal((T, Hq, 128)).astype(np.float32), dtype)
    q_start = np.concatenate([[0], np.cumsum(nqs)]).astype(np.int32)
    scale = float(np.float32(scale))
    ws = multi_query_workspace(pool, S, Hq, max(lens), max_q)
    out = torch.full_like(to_device_bits(q, dtype), float("nan"))
    pool.multi_query_attention(0, out, to_device_bits(q, dtype), torch.from_numpy(q_start).cuda(),
                               torch.from_numpy(tables).cuda(), torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda(),
                               max(lens), max_q, scale, workspace=ws,
                               host_context_lens=np.asarray(lens, dtype=np.int32))
    torch.cuda.synchronize()
    got = to_host_f64(out, dtype)
    for s in range(S):
        rows = slice(q_start[s], q_start[s + 1])
        ref = multi_query_one(host, 0, q[rows], tables[s], lens[s], scale, dtype)
        ok, st = within_tolerance(got[rows], ref, dtype)
        assert ok, (s, lens[s], nqs[s], st)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_multi_query_wide_path_table_beyond_lds(dtype):
    """A context whose table row exceeds the 2,048 entries the wide kernel
    caches in LDS (B = 8, 17,000 and 16,400 positions): its blocks are read
    from the table in memory instead.  Against the oracle, both launch
    orders, beside a short sequence that takes the cached path."""
    from oracle.decode import multi_query_one
    from paged_kv_cache_239_amd import multi_query_workspace
    G, Hkv, B, max_q = 4, 1, 8, 40
    _say(f"multi-query wide, long table, {dtype}")
    rng = np.random.default_rng(7300 + (dtype == "f16"))
    lens = [17000, 300, 16400]
    nqs = [40, 40, 33]
    S = len(lens)
    Hq = G * Hkv
    pool, host, tables, _ = _direct_case(rng, S, Hq, Hkv, B, dtype, lens)
    T = int(sum(nqs))
    q = round_to_dtype_bits(rng.standard_normal((T, Hq, 128)).astype(np.float32), dtype)
    q_start = np.concatenate([[0], np.cumsum(nqs)]).astype(np.int32)
    scale = float(np.float32(1 / np.sqrt(128)))
    ws = multi_query_workspace(pool, S, Hq, max(lens), max_q)
    dq = to_device_bits(q, dtype)
    outs = []
    for ordered in (False, True):
        out = torch.full_like(dq, float("nan"))
        pool.multi_query_attention(0, out, dq, torch.from_numpy(q_start).cuda(), torch.from_numpy(tables).cuda(),
                                   torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda(), max(lens), max_q, scale,
                                   workspace=ws, host_context_lens=np.asarray(lens, dtype=np.int32) if ordered else None)
        torch.cuda.synchronize()
        outs.append(out)
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    got = to_host_f64(outs[1], dtype)
    for s in range(S):
        rows = slice(q_start[s], q_start[s + 1])
        ref = multi_query_one(host, 0, q[rows], tables[s], lens[s], scale, dtype)
        ok, st = within_tolerance(got[rows], ref, dtype)
        assert ok, (s, lens[s], nqs[s], st)


def test_multi_query_one_query_each_matches_decode_within_tolerance():
    """nq = 1 everywhere: the multi-query path agrees with the oracle's decode
    (and so with pa_decode_attention) on the same inputs."""
    _say("multi-query with one query each")
    rng = np.random.default_rng(9)
    lens = [37, 91, 128, 201, 511]
    _mq_case(rng, 4, 2, 16, "f16", lens, [1] * len(lens))


def test_multi_query_workspace_bytes_monotone():
    from paged_kv_cache_239_amd import Pool
    pool = Pool(1, 8, 128, 16, 16, "bf16")
    lib = pool.lib
    sizes = [int(lib.pa_multi_query_workspace_bytes(pool.handle, S, 32, ctx, mq))
             for S, ctx, mq in [(4, 1000, 4), (4, 2000, 4), (8, 2000, 4), (8, 2000, 9), (8, 4000, 64)]]
    assert all(a <= b for a, b in zip(sizes, sizes[1:])) and sizes[0] > 0


@pytest.mark.parametrize("G,Hkv,B,dtype,max_q", [(1, 4, 16, "f16", 8), (2, 2, 32, "bf16", 4), (4, 2, 16, "bf16", 2),
                                                 (8, 1, 8, "f16", 1)])
def test_multi_query_vector_path_few_rows(G, Hkv, B, dtype, max_q):
    """At most 8 rows (query tokens x heads) per sequence: the vector path."""
    _say(f"multi-query vector path G={G} max_q={max_q}")
    rng = np.random.default_rng(500 + G)
    lens = [3, 40, 129, 700, 2049]
    nqs = [min(max_q, n) for n in [3, 1, max_q, 2, max_q]]
    _mq_case(rng, G, Hkv, B, dtype, lens, nqs)


@pytest.mark.parametrize("G,Hkv,B,dtype,max_q", [(1, 2, 16, "bf16", 20), (2, 2, 8, "f16", 12), (4, 2, 32, "bf16", 8),
                                                 (8, 1, 16, "f16", 4)])
def test_multi_query_matrix_path_16_rows(G, Hkv, B, dtype, max_q):
    """9 to 32 rows per sequence: the 16-row matrix-core path (waves split the context)."""
    _say(f"multi-query 16-row matrix path G={G} max_q={max_q}")
    rng = np.random.default_rng(700 + G)
    lens = [max_q, 40, 129, 1000, 2500]
    nqs = [max_q, 3, max_q, 1, max_q - 1]
    _mq_case(rng, G, Hkv, B, dtype, lens, nqs)


@pytest.mark.parametrize("G,Hkv,B,dtype,max_q", [(4, 2, 16, "bf16", 4), (1, 4, 32, "f16", 12), (2, 2, 8, "bf16", 6),
                                                 (8, 1, 64, "f16", 2)])
def test_multi_query_ordered_one_tile(G, Hkv, B, dtype, max_q):
    """9 to 16 rows per sequence (one matrix-core tile), partitions of equal
    length launched longest first from host copies of the lengths, against
    the oracle; also the same inputs in the fixed grid order."""
    _say(f"multi-query ordered G={G} max_q={max_q}")
    lens = [max_q, 40, 129, 1000, 2500, 1536, 4097, 700]
    nqs = [max_q, 1, max_q, 2, max_q - 1, max_q, max_q, 1]
    for ordered in (False, True):
        _mq_case(np.random.default_rng(900 + G), G, Hkv, B, dtype, lens, nqs, ordered=ordered)


# --------------------------------------------------------------------------------
# shared prefixes read once (grouped decode)
# --------------------------------------------------------------------------------
@pytest.mark.parametrize("B,fused", [(32, True), (32, False), (16, True), (8, True)])
def test_grouped_config2_prefix_sharing(B, fused):
    """Config 2's four prefix-sharing sequences form one run; full parity with
    the oracle over two steps, and the run is really used."""
    _say(f"grouped config 2 B={B} fused={fused}")
    wl, eng, st, results = _small_workload_step(2, steps=2, fused=fused, block_size=B, grouped=True)
    assert eng.max_shared > 0
    for got, ref, pairs in results:
        ok, stats = within_tolerance(got, ref, wl.cfg.dtype)
        assert ok, stats


@pytest.mark.parametrize("cfg,steps", [(5, 2), (6, 3)])
def test_grouped_full_size_sampled(cfg, steps):
    _full_size(cfg, steps=steps, layers=[0, 39], seqs_per_layer=8, seed=80 + cfg, grouped=True)


@pytest.mark.parametrize("short", [False, True])
@pytest.mark.parametrize("G,B,dtype", [(1, 16, "f16"), (2, 8, "bf16"), (4, 32, "bf16"), (8, 16, "f16")])
def test_grouped_direct_random_runs(G, B, dtype, short):
    """Random runs: sharing groups of 2-5 sequences with their own tails,
    singletons and unshared neighbours, NaN in every unused slot.  With
    `short`, no sequence has more than 128 positions beyond its run's shared
    prefix (members' tails and unshared sequences alike), as in a few steps
    of sampling after a fork."""
    _say(f"grouped direct G={G} B={B} {dtype} short={short}")
    rng = np.random.default_rng(1500 + G + B + (7 if short else 0))
    Hkv, d = 2, 128
    Hq = G * Hkv
    tables, lens = [], []
    nxt = 0
    # (members, shared prefix); None: an empty sequence (no positions; its
    # output row must still be written, as zeros)
    groups = [(3, 300), (1, 0), (2, 40), (5, 1100), (1, 0), (1, None), (1, 0), (4, 17), (1, None)]
    maxb = 0
    plan = []
    for size, prefix in groups:
        if prefix is None:
            tables.append([])
            lens.append(0)
            continue
        pref_blocks = -(-prefix // B) if prefix else 0
        pref = list(range(nxt, nxt + pref_blocks))
        nxt += pref_blocks
        for m in range(size):
            if short:
                n = prefix + int(rng.integers(1, min(3 * B, 64))) if prefix else int(rng.integers(1, 100))
            else:
                n = prefix + int(rng.integers(1, 3 * B)) if prefix else int(rng.integers(1, 900))
            if prefix % B:     # a partially filled shared block is copied before the sequence's own tokens
                own_from = pref_blocks - 1
            else:
                own_from = pref_blocks
            nb = -(-n // B)
            t = pref[:own_from] + list(range(nxt, nxt + nb - own_from))
            nxt += nb - own_from
            tables.append(t)
            lens.append(n)
            maxb = max(maxb, nb)
    P = nxt + 2
    perm = rng.permutation(P)
    S = len(lens)
    tab = np.full((S, maxb), 10 ** 6, dtype=np.int32)
    for s_, t in enumerate(tables):
        tab[s_, :len(t)] = perm[np.array(t, dtype=np.int64)]
    from paged_kv_cache_239_amd import Pool
    pool = Pool(1, Hkv, d, B, P, dtype)
    K = normal_bits(rng, (1, P, Hkv, B, d), dtype)
    V = normal_bits(rng, (1, P, Hkv, B, d), dtype)
    live = np.zeros((P, B), dtype=bool)
    for s_ in range(S):
        for t in range(lens[s_]):
            live[tab[s_, t // B], t % B] = True
    dead = np.broadcast_to(~live[:, None, :], (P, Hkv, B))
    K[0][dead] = dtype_nan_bits(dtype)
    V[0][dead] = dtype_nan_bits(dtype)
    pool.slab(0, "k").view(torch.int16).copy_(torch.from_numpy(K[0].view(np.int16)))
    pool.slab(0, "v").view(torch.int16).copy_(torch.from_numpy(V[0].view(np.int16)))
    host = HostPool.from_arrays(K, V)
    gs, gl, sg, mg, ms, max_suffix = pool.prefix_groups(tab, np.array(lens, dtype=np.int32))
    check_prefix_groups(tab.tolist(), lens, B, gs, gl, sg, mg, ms, max_suffix)
    assert ms > 0
    q = round_to_dtype_bits(rng.standard_normal((S, Hq, d)).astype(np.float32), dtype)
    scale = float(np.float32(1 / np.sqrt(d)))
    max_ctx = max(lens)
    if short:
        assert max_suffix <= 128 and ms <= 2048
    ws = torch.empty(pool.grouped_workspace_bytes(S, Hq, max_ctx, len(gl), mg, ms, max_suffix), dtype=torch.uint8,
                     device="cuda")
    dq = to_device_bits(q, dtype)
    ref = decode_layer(host, 0, q, tab, lens, scale, dtype)
    # the fixed grid, then the group pass longest first over equal partitions
    for hgl in (None, gl):
        out = torch.full_like(dq, float("nan"))
        pool.decode_attention_grouped(0, out, dq, torch.from_numpy(tab).cuda(),
                                      torch.tensor(lens, dtype=torch.int32, device="cuda"), max_ctx,
                                      torch.from_numpy(gs).cuda(), torch.from_numpy(gl).cuda(),
                                      torch.from_numpy(sg).cuda(), mg, ms, max_suffix, scale, ws, host_group_len=hgl)
        torch.cuda.synchronize()
        got = to_host_f64(out, dtype)
        ok, st = within_tolerance(got, ref, dtype)
        _say(f"ordered={hgl is not None} stats {st}")
        assert ok, st


# --------------------------------------------------------------------------------
# streaming-read ceiling kernel: reads exactly attention's key/value rows
# --------------------------------------------------------------------------------
@pytest.mark.parametrize("B,Hkv", [(8, 2), (16, 8), (32, 4), (64, 1), (128, 2)])
def test_stream_tiles_reads_exactly_the_attention_rows(B, Hkv):
    """The XOR of every 32-bit word pa_stream_tiles reads equals the XOR over
    the rows of positions 0..n-1 that the oracle gathers through the same
    tables (a row missed or read twice would change it), and each sequence's
    rows alone give that sequence's XOR (a call per sequence).  Lengths span
    ragged tails, zero and several thousand positions."""
    from oracle.cache_ops import gather
    _say(f"stream_tiles B={B} Hkv={Hkv}")
    rng = np.random.default_rng(4100 + B + Hkv)
    lens = [0, 1, 15, 16, 17, 1023, 1024, 1025, 2049, 3000, 77]
    S = len(lens)
    maxb = -(-max(lens) // B)
    P = sum(-(-n // B) for n in lens) + 3
    pool = _pool(1, Hkv, B, P, "bf16")
    bits = rng.integers(0, 2 ** 16, size=pool.nbytes // 2, dtype=np.uint16)
    pool.buffer.view(torch.int16).copy_(torch.from_numpy(bits.view(np.int16)))
    host = HostPool.from_arrays(bits.reshape(1, 2, P, Hkv, B, 128)[:, 0].copy(),
                                bits.reshape(1, 2, P, Hkv, B, 128)[:, 1].copy())
    perm = rng.permutation(P)
    tables = np.full((S, maxb), 10 ** 6, dtype=np.int32)
    nxt = 0
    for s, n in enumerate(lens):
        nb = -(-n // B)
        tables[s, :nb] = perm[nxt:nxt + nb]
        nxt += nb
    want_seq = []
    for s, n in enumerate(lens):
        Kc, Vc = gather(host, 0, tables[s], n)             # [n][Hkv][d] uint16
        words = np.concatenate([Kc.reshape(-1).view(np.uint32), Vc.reshape(-1).view(np.uint32)])
        want_seq.append(int(np.bitwise_xor.reduce(words)) if words.size else 0)
    want_all = 0
    for w in want_seq:
        want_all ^= w
    d_tab = torch.from_numpy(tables).cuda()
    d_len = torch.tensor(lens, dtype=torch.int32, device="cuda")
    chk = torch.zeros(1, dtype=torch.int32, device="cuda")
    pool.stream_tiles(0, d_tab, d_len, max(lens), chk)
    torch.cuda.synchronize()
    assert int(chk.cpu().numpy().view(np.uint32)[0]) == want_all
    for s, n in enumerate(lens):
        one = torch.zeros(1, dtype=torch.int32, device="cuda")
        pool.stream_tiles(0, d_tab[s:s + 1], d_len[s:s + 1], max(n, 1), one)
        torch.cuda.synchronize()
        assert int(one.cpu().numpy().view(np.uint32)[0]) == want_seq[s], (s, n)


# --------------------------------------------------------------------------------
# full size, every layer x every sequence of one step (oracle over all host cores)
# --------------------------------------------------------------------------------
def _every_layer(cfg, oracle_pool, ordered=True):
    from oracle.cache_ops import copy_blocks as o_copy, write_kv as o_write
    from oracle.replay import manager_step
    wl = with_headroom(make_workload(cfg), 1)
    c = wl.cfg
    eng = make_engine(wl, steps=1, ordered=ordered)
    _say(f"config {cfg} every layer: pool {eng.pool.nbytes / 2**30:.1f} GiB, S={wl.S}, L={c.L}, "
         f"oracle workers {oracle_pool.workers}")
    fill_pool_random(eng, wl)
    replay_history_device(eng, wl, write_values=False)
    # the oracle's starting slabs: torch's seeded fill, copied before any kernel writes
    snaps = {l: tuple(eng.pool.slab(l, w).clone() for w in ("k", "v")) for l in range(c.L)}
    st = build_state(wl, maxb=wl.max_blocks(1))
    qs, ks, vs = layer_inputs(wl, range(c.L), 0)
    outs = {l: torch.empty_like(qs[l]) for l in range(c.L)}
    max_ctx = eng.manager_step()
    eng.device_step(qs, ks, vs, outs, max_ctx, float(wl.scale))
    torch.cuda.synchronize()
    slots, pairs, lens = manager_step(st)
    assert list(eng.last_slots) == slots and list(eng.lens) == lens
    assert [tuple(p) for p in eng.last_pairs.tolist()] == pairs
    worst = 0.0
    for l in range(c.L):
        kd, vd = snaps.pop(l)
        K, V = oracle_pool.layer_buffer(tuple(kd.shape))
        torch.from_numpy(K.view(np.int16)).copy_(kd.view(torch.int16).cpu())
        torch.from_numpy(V.view(np.int16)).copy_(vd.view(torch.int16).cpu())
        del kd, vd
        hp = HostPool.from_arrays(K[None], V[None])
        o_copy(hp, pairs)
        o_write(hp, 0, wl.knew_bits(l, 0), wl.vnew_bits(l, 0), slots)
        # the device's cache after the step's writes equals the oracle's, byte for byte
        assert np.array_equal(to_host_bits(eng.pool.slab(l, "k")), K)
        assert np.array_equal(to_host_bits(eng.pool.slab(l, "v")), V)
        ref, wall, _ = oracle_pool.decode_layer(wl.q_bits(l, 0), st.tables, st.lens, float(wl.scale), c.dtype)
        got = to_host_f64(outs[l], c.dtype)
        ok, stats = within_tolerance(got, ref, c.dtype)
        assert ok, (cfg, l, stats)
        worst = max(worst, stats["max_abs"])
        _say(f"config {cfg} layer {l}: {wl.S} sequences in {wall:.1f} s, max_abs {stats['max_abs']:.2e}")
    _say(f"config {cfg}: all {c.L} layers x {wl.S} sequences within tolerance, worst max_abs {worst:.2e}")
    del eng
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_config3_every_layer_every_sequence(oracle_pool):
    _every_layer(3, oracle_pool)


@pytest.mark.timeout(900)
def test_config4_every_layer_every_sequence(oracle_pool):
    _every_layer(4, oracle_pool)


def test_config5_fork_step_cow_sources_unchanged_debug_engine():
    """The fork step of the parallel-sampling workload with the engine in
    debug mode (pa_validate_step on every step).  Three of a prompt's four
    branches copy its partial last block; the fourth then finds the count at
    one and writes in place.  After the copies and the fused writes, in every
    layer: every copy equals its source except the one row per (key or
    value, head) that its own branch writes, and every source block differs
    from its former contents only in the row written in place, if any."""
    _say("config 5 fork step, debug engine, copy-on-write sources")
    wl = with_headroom(make_workload(5), 1)
    c = wl.cfg
    eng = make_engine(wl, steps=1, grouped=True)
    eng.debug = True
    fill_pool_random(eng, wl)
    replay_history_device(eng, wl, write_values=False)
    qs, ks, vs = layer_inputs(wl, range(c.L), 0)
    outs = {l: torch.empty_like(qs[l]) for l in range(c.L)}
    max_ctx = eng.manager_step()
    pairs = eng.last_pairs.copy()
    assert len(pairs) > 100
    tile = eng.pool.nbytes // (2 * c.L * wl.P)
    view = eng.pool.buffer.view(2 * c.L, wl.P, tile)
    srcs = sorted(set(pairs[:, 0].tolist()))
    src_idx = torch.tensor(srcs, dtype=torch.int64, device="cuda")
    dst_idx = torch.from_numpy(pairs[:, 1].astype(np.int64)).cuda()
    before = view.index_select(1, src_idx).clone()
    eng.device_step(qs, ks, vs, outs, max_ctx, float(wl.scale))
    torch.cuda.synchronize()
    written = {}                                  # block -> rows the step writes into it
    for slot in eng.last_slots.tolist():
        written.setdefault(int(slot) // c.B, []).append(int(slot) % c.B)
    row = c.d * 2

    def changed_rows(a, b):                       # [2L][n][tile] pair -> per block, rows that differ anywhere
        d = (a.view(2 * c.L, a.shape[1], c.Hkv, c.B, row) != b.view(2 * c.L, b.shape[1], c.Hkv, c.B, row))
        return d.any(dim=-1).any(dim=0).any(dim=1).cpu().numpy()      # [n][B]

    after_src = view.index_select(1, src_idx)
    diff = changed_rows(after_src, before)
    for i, b in enumerate(srcs):
        assert np.nonzero(diff[i])[0].tolist() == sorted(written.get(b, [])), b
    pos = {b: i for i, b in enumerate(srcs)}
    dst = view.index_select(1, dst_idx)
    src_before = before.index_select(1, torch.tensor([pos[a] for a in pairs[:, 0].tolist()], device="cuda"))
    diff = changed_rows(dst, src_before)
    for i, (a, b) in enumerate(pairs.tolist()):
        assert np.nonzero(diff[i])[0].tolist() == sorted(written[b]), (a, b)
    in_place = sum(1 for b in srcs if b in written)
    _say(f"{len(pairs)} copies of {len(srcs)} blocks checked over {c.L} layers; {in_place} sources written in place")
