"""Shared helpers of the GPU tests, smoke() and bench: build a decode engine
for a workload, fill its pool, and compare device results with the oracle.

The device side is driven only through the product binding
(paged_kv_cache_239_amd); expected values come only from ``oracle``; both
take their inputs from ``workloads``.
"""

from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np

from oracle.cache_ops import HostPool, copy_blocks, write_kv
from oracle.decode import decode_one
from oracle.replay import beam_reorder, build_state, manager_step
from workloads import make_workload
from workloads.gen import dtype_nan_bits

ATOL = 2e-3
RTOL = 1e-2
REL_FLOOR = ATOL / RTOL   # 0.2: below it the absolute bound is the binding one


def tol_stats(out: np.ndarray, ref: np.ndarray) -> Dict[str, float]:
    """max_abs over all elements, max_abs_small over |ref| < 0.2, max_rel over
    |ref| >= 0.2, and the worst allclose margin |o-r| - (2e-3 + 1e-2 |r|)."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(out - ref)
    big = np.abs(ref) >= REL_FLOOR
    max_rel = float(np.max(err[big] / np.abs(ref[big]))) if np.any(big) else 0.0
    small = ~big
    return {
        "max_abs": float(np.max(err)) if err.size else 0.0,
        "max_abs_small": float(np.max(err[small])) if np.any(small) else 0.0,
        "max_rel": max_rel,
        "allclose_worst": float(np.max(err - (ATOL + RTOL * np.abs(ref)))) if err.size else -1.0,
        "finite": bool(np.all(np.isfinite(out))),
    }


def within_tolerance(out, ref) -> Tuple[bool, Dict[str, float]]:
    """Absolute bound 2e-3 where |ref| < 0.2, relative bound 1e-2 where
    |ref| >= 0.2 (the two agree at 0.2 = 2e-3 / 1e-2).  Above 0.5 the
    absolute bound alone would be below half an ulp of a bf16 output."""
    st = tol_stats(out, ref)
    ok = st["finite"] and st["max_abs_small"] <= ATOL and st["max_rel"] <= RTOL
    return ok, st


def to_device_bits(bits: np.ndarray, dtype: str, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    t = t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)
    return t.to(device)


def to_host_f64(t, dtype: str) -> np.ndarray:
    import torch
    bits = t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    from oracle.dtypes import bits_to_f64
    return bits_to_f64(bits, dtype)


def to_host_bits(t) -> np.ndarray:
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def make_engine(wl, steps: int = 1, device="cuda", fused: bool = True, grouped: bool = False,
                ordered: bool = True):
    from paged_kv_cache_239_amd.engine import DecodeEngine
    c = wl.cfg
    return DecodeEngine(c.L, c.Hq, c.Hkv, c.d, c.B, wl.P, c.dtype, wl.S, wl.max_blocks(steps),
                        free_order=wl.free_order, device=device, fused=fused, grouped=grouped, ordered=ordered)


def replay_history_device(eng, wl, write_values: bool) -> None:
    """Run the workload's history through the native manager; with
    ``write_values`` the prefill keys/values are written with pa_write_kv
    (copies first, if any)."""
    import torch
    c = wl.cfg
    for op_index, op in enumerate(wl.history):
        if op[0] == "append":
            _, s, ntok = op
            slots, pairs = eng.append(s, ntok)
            if write_values and ntok:
                if pairs:
                    eng.pool.copy_blocks(torch.tensor(pairs, dtype=torch.int32, device=eng.device))
                d_slots = torch.from_numpy(np.asarray(slots, dtype=np.int64)).to(eng.device)
                for layer in range(c.L):
                    k = to_device_bits(wl.prefill_bits(layer, op_index, ntok, "k"), c.dtype, eng.device)
                    v = to_device_bits(wl.prefill_bits(layer, op_index, ntok, "v"), c.dtype, eng.device)
                    eng.pool.write_kv(layer, k, v, d_slots)
        else:
            _, child, parent, ntok = op
            eng.fork(child, parent, ntok)
    eng.upload_tables()


def fill_pool_nan(eng, dtype: str) -> None:
    import torch
    bits = dtype_nan_bits(dtype)
    eng.pool.buffer.view(torch.int16).fill_(bits if bits < 0x8000 else bits - 0x10000)


def fill_pool_random(eng, wl) -> None:
    """Seeded N(0,1) in every slot of every layer (device RNG)."""
    import torch
    for layer in range(wl.cfg.L):
        for which in ("k", "v"):
            g = torch.Generator(device=eng.device)
            g.manual_seed(wl.pool_fill_seed(layer, which))
            eng.pool.slab(layer, which).normal_(generator=g)


def layer_inputs(wl, layers: Sequence[int], step: int, device="cuda"):
    c = wl.cfg
    qs, ks, vs = {}, {}, {}
    for layer in layers:
        qs[layer] = to_device_bits(wl.q_bits(layer, step), c.dtype, device)
        ks[layer] = to_device_bits(wl.knew_bits(layer, step), c.dtype, device)
        vs[layer] = to_device_bits(wl.vnew_bits(layer, step), c.dtype, device)
    return qs, ks, vs


def snapshot_layers(eng, layers: Sequence[int]) -> Dict[int, HostPool]:
    """Host copy of whole layer slabs (device pool contents that torch's
    generator wrote), one single-layer oracle pool per layer."""
    out = {}
    for layer in layers:
        K = to_host_bits(eng.pool.slab(layer, "k"))[None]
        V = to_host_bits(eng.pool.slab(layer, "v"))[None]
        out[layer] = HostPool.from_arrays(K, V)
    return out


class OracleSide:
    """The oracle's own view of a large workload: its manager replays the
    history; for the sampled layers it holds host pools that start from the
    snapshot and receive the oracle's own copies and writes."""

    def __init__(self, wl, snapshots: Dict[int, HostPool], maxb: int):
        self.wl = wl
        self.state = build_state(wl, maxb=maxb)
        self.pools = snapshots

    def step(self, step: int):
        if self.wl.cfg.beam:
            beam_reorder(self.state, self.wl.parents(step))
        slots, pairs, lens = manager_step(self.state)
        for layer, pool in self.pools.items():
            copy_blocks(pool, pairs)
            write_kv(pool, 0, self.wl.knew_bits(layer, step), self.wl.vnew_bits(layer, step), slots)
        return slots, pairs, lens

    def expected(self, layer: int, s: int, step: int) -> np.ndarray:
        c = self.wl.cfg
        q = self.wl.q_bits(layer, step)[s]
        return decode_one(self.pools[layer], 0, q, self.state.tables[s], self.state.lens[s],
                          float(self.wl.scale), c.dtype)
