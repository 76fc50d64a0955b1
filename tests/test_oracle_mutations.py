"""Planted mistakes in the oracle must fail at least one pin.

Each case swaps one oracle function for a plausibly wrong variant (wrong
head mapping, dropped scale, no max shift, swapped block/offset index, a
missing decref, a missing copy) and runs the pins that should notice.  The
mistakes live only here, on the CPU, inside monkeypatch scopes.
"""

import numpy as np
import pytest

import oracle.attention as att
import oracle.cache_ops as cops
import oracle.decode as dec
import oracle.manager as man
from tests import test_oracle_attention as TA
from tests import test_oracle_cache as TC
from tests import test_oracle_manager as TM


def _fails(fn):
    try:
        fn()
    except (AssertionError, FloatingPointError, ValueError, IndexError, man.ManagerError):
        return True
    return False


def _dense_wrong_head(q, K, V, scale):
    q = np.asarray(q, np.float64); K = np.asarray(K, np.float64); V = np.asarray(V, np.float64)
    Hq, d = q.shape
    Hkv = K.shape[1]
    out = np.zeros((Hq, d))
    if K.shape[0] == 0:
        return out
    for h in range(Hq):
        k = h % Hkv                                   # interleaved instead of grouped
        p = att.softmax_weights(scale * (K[:, k, :] @ q[h]))
        out[h] = p @ V[:, k, :]
    return out


def _dense_no_scale(q, K, V, scale):
    return _orig_dense(q, K, V, 1.0)


def _softmax_no_shift(s):
    s = np.asarray(s, np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        e = np.exp(s)
        return e / np.sum(e)


def _gather_swapped(pool, layer, table, n):
    B = pool.B
    Kc = np.empty((n, pool.Hkv, pool.d), dtype=np.uint16)
    Vc = np.empty((n, pool.Hkv, pool.d), dtype=np.uint16)
    for t in range(n):
        blk = int(table[min(t % B, len(table) - 1)])
        Kc[t] = pool.K[layer, blk, :, t // B % B, :]
        Vc[t] = pool.V[layer, blk, :, t // B % B, :]
    return Kc, Vc


def _copy_keys_only(pool, pairs):
    for src, dst in pairs:
        pool.K[:, int(dst)] = pool.K[:, int(src)]


_orig_dense = att.dense_attention


def test_wrong_head_mapping_is_caught(monkeypatch):
    monkeypatch.setattr(att, "dense_attention", _dense_wrong_head)
    monkeypatch.setattr(TA, "dense_attention", _dense_wrong_head)
    assert _fails(TA.test_gqa_equals_mha_with_repeated_kv_heads) or \
        _fails(TA.test_matches_torch_sdpa_float64)


def test_dropped_scale_is_caught(monkeypatch):
    monkeypatch.setattr(TA, "dense_attention", _dense_no_scale)
    assert _fails(TA.test_matches_torch_sdpa_float64)


def test_missing_max_shift_is_caught(monkeypatch):
    monkeypatch.setattr(att, "softmax_weights", _softmax_no_shift)
    monkeypatch.setattr(TA, "softmax_weights", _softmax_no_shift)
    assert _fails(lambda: TA.test_extreme_logits_no_overflow(1e4))


def test_swapped_block_and_offset_is_caught(monkeypatch):
    monkeypatch.setattr(cops, "gather", _gather_swapped)
    monkeypatch.setattr(TC, "gather", _gather_swapped)
    monkeypatch.setattr(dec, "gather", _gather_swapped)
    assert _fails(TC.test_write_then_gather_roundtrip_and_skip)


def test_partial_copy_is_caught(monkeypatch):
    monkeypatch.setattr(cops, "copy_blocks", _copy_keys_only)
    monkeypatch.setattr(TC, "copy_blocks", _copy_keys_only)
    assert _fails(TC.test_copy_blocks_whole_block_every_layer)


def test_cow_without_decref_is_caught(monkeypatch):
    orig = man.BlockManager.append_slot

    def bad_append(self, table, n_before):
        idx, off = divmod(n_before, self.B)
        if off and self.ref[table[idx]] > 1:
            old = table[idx]
            new = self.alloc()
            table[idx] = new                      # forgets to drop the old count
            return new * self.B + off, (old, new)
        return orig(self, table, n_before)

    monkeypatch.setattr(man.BlockManager, "append_slot", bad_append)
    assert _fails(TM.test_copy_on_write_shared_partial_block)
    assert any(_fails(lambda s=s: TM.test_random_traces_keep_invariants(s)) for s in range(6))


def test_lifo_free_list_is_caught(monkeypatch):
    def bad_decref(self, blk):
        self._check(blk)
        if self.ref[blk] == 0:
            raise man.InvalidArg("free")
        self.ref[blk] -= 1
        if self.ref[blk] == 0:
            self.free.appendleft(blk)             # reuses the address at once

    monkeypatch.setattr(man.BlockManager, "decref", bad_decref)
    assert _fails(TM.test_fifo_free_list_and_release)
