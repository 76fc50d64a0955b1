"""Seeded random draws for the decode workloads.

Every draw comes from ``numpy.random.default_rng((239, cfg, layer, purpose,
step))`` so any single layer or step can be regenerated on its own.  Values
are N(0, 1) in float32 rounded to the storage dtype with round-to-nearest-even,
and are handed around as raw 16-bit patterns (``uint16``) so that both sides
start from identical bits.

The sequence history is described abstractly (which sequence receives how
many prefill tokens, which sequence maps which other sequence's leading
blocks); each side replays it with its own block manager.
"""

from __future__ import annotations

import dataclasses
import math
import re
from dataclasses import dataclass
from typing import List, Tuple

import numpy as np

from .configs import FIVE_LENGTHS, DecodeConfig, get_config

# purpose codes for the seed tuple
P_LENGTHS = 1
P_PERM = 2
P_Q = 3
P_KNEW = 4
P_VNEW = 5
P_PREFILL_K = 6
P_PREFILL_V = 7
P_POOL_K = 8
P_POOL_V = 9
P_PARENTS = 10

SEED_ROOT = 239


def rng_for(cfg_id: int, layer: int, purpose: int, step: int = 0) -> np.random.Generator:
    return np.random.default_rng((SEED_ROOT, int(cfg_id), int(layer), int(purpose), int(step)))


def seed_int(cfg_id: int, layer: int, purpose: int, step: int = 0) -> int:
    """A 63-bit integer seed derived from the same tuple (for device RNGs)."""
    ss = np.random.SeedSequence((SEED_ROOT, int(cfg_id), int(layer), int(purpose), int(step)))
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64(0x7FFF_FFFF_FFFF_FFFF))


def round_to_dtype_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> 16-bit storage pattern, round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        u = x.view(np.uint32).astype(np.uint64)
        nan = np.isnan(x)
        r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        r = r.astype(np.uint16)
        r[nan] = 0x7FC0
        return r
    raise ValueError(dtype)


def dtype_nan_bits(dtype: str) -> int:
    return 0x7E00 if dtype == "f16" else 0x7FC0


def normal_bits(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    return round_to_dtype_bits(rng.standard_normal(size=shape, dtype=np.float32), dtype)


@dataclass
class Workload:
    """One decode workload: shapes, lengths, pool, history and value recipes."""

    cfg: DecodeConfig
    lengths0: np.ndarray        # int64 [S]: context length at decode step 0 (incl. new token)
    P: int                      # physical blocks in the pool
    free_order: np.ndarray      # int32 [P]: initial free-list order (a permutation)
    history: List[Tuple]        # abstract prefill/sharing ops, replayed by each side
    scale: np.float32           # softmax scale 1/sqrt(d), as the float32 both sides use

    @property
    def S(self) -> int:
        return int(self.lengths0.shape[0])

    def lengths_at(self, step: int) -> np.ndarray:
        return self.lengths0 + int(step)

    def max_blocks(self, steps: int | None = None) -> int:
        """Block-table width that holds every sequence after ``steps`` decode steps."""
        steps = self.cfg.steps if steps is None else steps
        B = self.cfg.B
        return int(-(-int(self.lengths0.max() + steps - 1) // B))

    # ---- per-layer values -------------------------------------------------
    def q_bits(self, layer: int, step: int = 0) -> np.ndarray:
        c = self.cfg
        return normal_bits(rng_for(c.cfg_id, layer, P_Q, step), (self.S, c.Hq, c.d), c.dtype)

    def knew_bits(self, layer: int, step: int = 0) -> np.ndarray:
        c = self.cfg
        return normal_bits(rng_for(c.cfg_id, layer, P_KNEW, step), (self.S, c.Hkv, c.d), c.dtype)

    def vnew_bits(self, layer: int, step: int = 0) -> np.ndarray:
        c = self.cfg
        return normal_bits(rng_for(c.cfg_id, layer, P_VNEW, step), (self.S, c.Hkv, c.d), c.dtype)

    def prefill_bits(self, layer: int, op_index: int, ntok: int, which: str) -> np.ndarray:
        """Logical K or V of the ``ntok`` tokens that history op ``op_index``
        appends: [ntok][Hkv][d], one seeded stream per (layer, op)."""
        c = self.cfg
        purpose = P_PREFILL_K if which == "k" else P_PREFILL_V
        return normal_bits(rng_for(c.cfg_id, layer, purpose, op_index), (ntok, c.Hkv, c.d), c.dtype)

    def parents(self, step: int) -> np.ndarray:
        """Beam workloads: int32 [S], the old sequence each new sequence
        continues at ``step``.  Per prompt, W draws from its W beams with
        probabilities proportional to W, W-1, ..., 1 (beam j of a prompt
        stands for its j-th best candidate), sorted, so a prompt's beams stay
        together and some beams end while others split."""
        c = self.cfg
        W = c.branches
        r = rng_for(c.cfg_id, 0, P_PARENTS, step)
        w = np.arange(W, 0, -1, dtype=np.float64)
        draws = r.choice(W, size=(c.prompts, W), p=w / w.sum())
        draws.sort(axis=1)
        return (np.arange(c.prompts)[:, None] * W + draws).reshape(-1).astype(np.int32)

    def pool_fill_seed(self, layer: int, which: str) -> int:
        """Seed for filling a whole layer slab in device memory (large workloads)."""
        return seed_int(self.cfg.cfg_id, layer, P_POOL_K if which == "k" else P_POOL_V)


def _lengths(c: DecodeConfig) -> np.ndarray:
    if c.length_kind == "five":
        return np.array(FIVE_LENGTHS, dtype=np.int64)
    if c.length_kind == "uniform":
        r = rng_for(c.cfg_id, 0, P_LENGTHS)
        return r.integers(c.uniform_lo, c.uniform_hi, size=c.S, endpoint=True).astype(np.int64)
    if c.length_kind == "fixed":
        return np.full(c.S, c.fixed_len, dtype=np.int64)
    if c.length_kind == "lognormal_branches":
        r = rng_for(c.cfg_id, 0, P_LENGTHS)
        z = r.standard_normal(size=c.prompts)
        prompt = np.rint(np.exp(math.log(c.lognormal_median) + c.lognormal_sigma * z))
        prompt = np.clip(prompt, 1, c.max_len - c.steps).astype(np.int64)
        # every branch has its prompt's length; step 0 adds the first new token
        return np.repeat(prompt, c.branches) + 1
    raise ValueError(c.length_kind)


def _ceil_div(a, b):
    return -(-a // b)


def _pool_blocks(c: DecodeConfig, lengths0: np.ndarray) -> int:
    B = c.B
    if c.pool_kind == "fixed":
        return int(c.pool_blocks)
    used = int(np.sum(_ceil_div(lengths0, B)))
    if c.pool_kind == "scaled":
        return int(math.ceil(c.pool_scale * used))
    if c.pool_kind == "exact":
        return used
    if c.pool_kind == "branch_bound":
        prompt = lengths0[:: c.branches] - 1
        shared = int(np.sum(_ceil_div(prompt, B)))
        # per branch: one copy-on-write of the prompt's last block plus the
        # blocks that `steps` new tokens can open
        return shared + c.S * (int(_ceil_div(c.steps, B)) + 1)
    raise ValueError(c.pool_kind)


def _history(c: DecodeConfig, lengths0: np.ndarray) -> List[Tuple]:
    """Abstract ops, replayed in order by each side's manager:
    ("append", seq, ntok)            -- prefill ntok tokens onto seq
    ("fork", child, parent, ntok)    -- child maps parent's first ceil(ntok/B)
                                        blocks; child length becomes ntok
    After the history, every sequence holds lengths0[s] - 1 tokens."""
    ops: List[Tuple] = []
    S = len(lengths0)
    if c.length_kind == "lognormal_branches":
        for p in range(c.prompts):
            root = p * c.branches
            n = int(lengths0[root]) - 1
            ops.append(("append", root, n))
            for b in range(1, c.branches):
                ops.append(("fork", root + b, root, n))
        return ops
    if c.share_prefix_tokens:
        # Sequence 1 writes the shared prefix (its first two blocks); sequence 0
        # maps both blocks but sees only its own shorter prefix, so its next
        # write lands inside the shared partial block; sequences 2 and 3 map
        # the whole prefix.  Both prefix blocks end at refcount 4.
        shared = c.share_prefix_tokens
        ops.append(("append", 1, shared))
        ops.append(("fork", 0, 1, int(lengths0[0]) - 1))
        ops.append(("fork", 2, 1, shared))
        ops.append(("fork", 3, 1, shared))
        for s in (1, 2, 3):
            ops.append(("append", s, int(lengths0[s]) - 1 - shared))
        for s in range(4, S):
            ops.append(("append", s, int(lengths0[s]) - 1))
        return ops
    for s in range(S):
        ops.append(("append", s, int(lengths0[s]) - 1))
    return ops


def with_headroom(wl: Workload, steps: int) -> Workload:
    """The same workload with its pool extended, if needed, so that every
    sequence can take ``steps`` more tokens without sharing (for running many
    decode steps over a workload whose pool is sized exactly).  Extra block
    ids follow the original free order in a seeded shuffled order."""
    c = wl.cfg
    B = c.B
    if c.pool_kind == "branch_bound":
        shared = int(np.sum(_ceil_div(wl.lengths0[:: c.branches] - 1, B)))
        need = shared + wl.S * (int(_ceil_div(steps, B)) + 1)
    else:
        need = int(np.sum(_ceil_div(wl.lengths0 - 1 + steps, B)))
    if need <= wl.P:
        return wl
    extra = np.arange(wl.P, need, dtype=np.int32)
    extra = extra[rng_for(wl.cfg.cfg_id, 0, P_PERM, 1).permutation(len(extra))]
    return Workload(cfg=wl.cfg, lengths0=wl.lengths0, P=need,
                    free_order=np.concatenate([wl.free_order, extra]).astype(np.int32),
                    history=wl.history, scale=wl.scale)


def _at_block_size(c: DecodeConfig, B: int, lengths0: np.ndarray) -> DecodeConfig:
    """``c`` at block size ``B``; seeds, lengths and values are unchanged.  A
    fixed pool keeps its ratio of pool blocks to used blocks (rounded up)."""
    name = re.sub(r"_b\d+", f"_b{B}", c.name, count=1)
    if name == c.name:
        name = f"{c.name}_b{B}"
    kw = {"B": int(B), "name": name}
    if c.pool_kind == "fixed":
        used_old = int(np.sum(_ceil_div(lengths0, c.B)))
        used_new = int(np.sum(_ceil_div(lengths0, B)))
        kw["pool_blocks"] = int(_ceil_div(int(c.pool_blocks) * used_new, used_old))
    return dataclasses.replace(c, **kw)


def _head_shard(c: DecodeConfig, n: int) -> DecodeConfig:
    """One GPU's share of ``c`` when its heads are split over ``n`` GPUs:
    Hq / n query heads and Hkv / n key/value heads (a query group stays with
    its key/value head); sequences, lengths, history and seeds unchanged."""
    if n < 1 or c.Hkv % n:
        raise ValueError(f"{n} shards do not divide {c.Hkv} key/value heads")
    return dataclasses.replace(c, Hq=c.Hq // n, Hkv=c.Hkv // n, name=f"{c.name}_heads1of{n}",
                               description=f"{c.description}; one GPU's share with the heads split over {n} "
                                           f"GPUs: {c.Hq // n} query / {c.Hkv // n} KV heads")


def make_workload(cfg_id: int, block_size: int | None = None, head_shards: int = 1) -> Workload:
    """Workload ``cfg_id``; ``block_size`` runs the same sequences, history and
    values over blocks of another size; ``head_shards`` > 1 keeps one GPU's
    share of the heads."""
    c = get_config(cfg_id)
    lengths0 = _lengths(c)
    if block_size is not None and int(block_size) != c.B:
        c = _at_block_size(c, int(block_size), lengths0)
    if int(head_shards) != 1:
        c = _head_shard(c, int(head_shards))
    assert lengths0.shape[0] == c.S
    P = _pool_blocks(c, lengths0)
    perm = rng_for(c.cfg_id, 0, P_PERM).permutation(P).astype(np.int32)
    return Workload(cfg=c, lengths0=lengths0, P=P, free_order=perm,
                    history=_history(c, lengths0),
                    scale=np.float32(1.0 / math.sqrt(c.d)))
