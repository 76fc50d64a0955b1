#!/usr/bin/env python3
"""Decode-step benchmark of the paged key/value cache on one MI355X.

Workload (default): GQA decode, 32 layers run in sequence, 32 query / 8
key-value heads, head dim 128, bf16, batch 64 with context lengths uniform in
[512, 4096], block size 16, pool of 1.25x the used blocks with shuffled
physical blocks.  A step is the whole path for one new token per sequence:
host block manager (slots, copy-on-write pairs), upload of tables, block
copies, then for every layer the cache write of the new token and the paged
decode attention.  Inputs are seeded synthetic values resident in device
memory before timing starts.

Prints one JSON line: whole-step throughput in algorithmic GB/s (cache bytes
the method must move: the useful key/value positions, queries, outputs,
tables, and the written and copied bytes), seq-steps/s, the roofline of the
attention kernel (HIP events around every launch in the timed region), and
the fp64 CPU oracle timed on a bounded sample of the same step.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published
# the attention kernel's sources: a counter record applies only to these exact files
KERNEL_SOURCES = [os.path.join(ROOT, "paged_kv_cache_239_amd", "csrc", f)
                  for f in ("pa_attention.hip", "pa_device_common.h")]
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_sha() -> str:
    import hashlib
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(here: dict):
    """HBM bytes per attention call from a committed rocprofv3 counter
    summary (profiles/*_pmc.md, a JSON record each) taken on this workload
    and launch mode (``here``) and on this version of the kernel source, or
    None when there is none."""
    import glob
    sha = kernel_source_sha()
    for path in sorted(glob.glob(os.path.join(PROFILES, "*_pmc.md"))):
        try:
            text = open(path).read()
            rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
        except (OSError, IndexError, ValueError):
            continue
        if rec.get("kernel_source_sha256") == sha and rec.get("workload") == here:
            return rec
    return None


class HipEvents:
    """Timing-only HIP events (hipEventDisableSystemFence): recording them adds
    no cache write-back between the kernels they bracket.  torch's events use
    the default flags, whose system-scope fence costs several microseconds
    per record on this GPU."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        self.C = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = []

    def create(self):
        e = self.C.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(self.C.byref(e), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")
        self.events.append(e)
        return e

    def record(self, e, stream_handle):
        rc = self.hip.hipEventRecord(e, self.C.c_void_p(stream_handle))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def elapsed_ms(self, a, b) -> float:
        ms = self.C.c_float()
        rc = self.hip.hipEventElapsedTime(self.C.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(ms.value)

    def close(self):
        for e in self.events:
            self.hip.hipEventDestroy(e)
        self.events = []


def attn_bytes(lens, S, Hq, Hkv, d, B, b=2) -> int:
    """Algorithmic bytes of one layer's decode attention."""
    lens = np.asarray(lens, dtype=np.int64)
    kv = int(np.sum(lens)) * 2 * Hkv * d * b
    qo = 2 * S * Hq * d * b
    meta = int(np.sum((lens + B - 1) // B)) * 4 + S * 4
    return kv + qo + meta


def unique_kv_bytes(tables, lens, c, P) -> int:
    """Key/value bytes of one layer counted once per physical block: the
    largest number of positions any sequence reads from that block."""
    lens = np.asarray(lens, dtype=np.int64)
    j = np.arange(tables.shape[1], dtype=np.int64)
    valid = j[None, :] < ((lens + c.B - 1) // c.B)[:, None]
    pos = np.minimum(c.B, lens[:, None] - j[None, :] * c.B)
    best = np.zeros(P, dtype=np.int64)
    np.maximum.at(best, tables[valid].astype(np.int64), pos[valid])
    return int(best.sum()) * 2 * c.Hkv * c.d * 2


def write_bytes(S, Hkv, d, b=2) -> int:
    return 2 * (2 * S * Hkv * d * b) + 8 * S


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 100; for a workload of several decode steps, its own "
                         "steps after the first)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before (default: 5; 1 -- the fork step -- for a workload of "
                         "several decode steps)")
    ap.add_argument("--config", type=int, default=3, help="workload id (3 = the GQA 32/8 workload)")
    ap.add_argument("--block-size", type=int, default=0,
                    help="store the workload in blocks of this many tokens (8, 16, 32, 64 or 128; "
                         "default: the workload's own)")
    ap.add_argument("--head-shards", type=int, default=1, metavar="N",
                    help="run one GPU's share of the workload when its heads are split over N GPUs "
                         "(Hq / N and Hkv / N heads, same sequences)")
    ap.add_argument("--swap", type=int, default=0, metavar="N",
                    help="instead of decode steps: swap the first N sequences of the workload out to a "
                         "pinned host pool and back, and time it")
    ap.add_argument("--queries", type=int, default=0, metavar="Q",
                    help="instead of one token per sequence: every step appends Q tokens per sequence "
                         "(speculative verification, chunked prefill) and runs multi-query attention")
    ap.add_argument("--grouped", choices=["auto", "on", "off"], default="auto",
                    help="read prefixes that several sequences share once per group (auto: for the "
                         "workloads whose sequences share prompt blocks)")
    ap.add_argument("--order", choices=["on", "off"], default="on",
                    help="launch the context partitions longest first from the manager's lengths "
                         "(pa_decode_attention_ordered); off: the fixed grid order")
    ap.add_argument("--cpu-baseline", choices=["on", "off"], default="on")
    ap.add_argument("--cpu-layers", type=int, default=0,
                    help="layers the oracle checks on the final step (default: all), evenly spaced")
    ap.add_argument("--dump", default="", help="write per-step and per-launch times (JSON) here")
    ap.add_argument("--calibrate", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times (reference for "
                         "hardware byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the library has no "
                                   "multi-GPU path (each GPU would hold its own shard of heads "
                                   "or sequences with no exchange inside attention; --head-shards N "
                                   "runs one GPU's share)",
                          "n_gpus": args.gpus}))
        return 2

    # The oracle's worker processes start before this process touches the GPU.
    opool = None
    if args.cpu_baseline == "on" and not (args.calibrate or args.swap or args.queries):
        from oracle.parallel import OraclePool
        opool = OraclePool()
    try:
        return run(args, opool)
    finally:
        if opool is not None:
            opool.close()


def run(args, opool) -> int:
    import torch

    from paged_kv_cache_239_amd.engine import DecodeEngine
    from workloads import make_workload, with_headroom

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        return 1
    torch.cuda.set_device(0)
    if args.calibrate:
        src = torch.ones(1 << 28, dtype=torch.int32, device="cuda")      # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": src.numel() * 4, "copies": 3}))
        return 0

    if args.swap:
        return swap_bench(args)
    if args.queries:
        return multi_query_bench(args)

    from workloads import get_config
    steps_of = get_config(args.config).steps
    W = args.warmup if args.warmup is not None else (1 if steps_of > 1 else 5)
    K = args.steps if args.steps is not None else (steps_of - W if steps_of > 1 else 100)
    wl = with_headroom(make_workload(args.config, block_size=args.block_size or None,
                                     head_shards=args.head_shards), W + K + 1)
    c = wl.cfg
    grouped = args.grouped == "on" or (args.grouped == "auto" and c.length_kind == "lognormal_branches")
    eng = DecodeEngine(c.L, c.Hq, c.Hkv, c.d, c.B, wl.P, c.dtype, wl.S, wl.max_blocks(W + K),
                       free_order=wl.free_order, grouped=grouped, ordered=args.order == "on")
    # seeded N(0,1) pool contents (device RNG), then the prefill history on the native manager
    for layer in range(c.L):
        for which in ("k", "v"):
            g = torch.Generator(device="cuda")
            g.manual_seed(wl.pool_fill_seed(layer, which))
            eng.pool.slab(layer, which).normal_(generator=g)
    for op in wl.history:
        if op[0] == "append":
            eng.append(op[1], op[2])
        else:
            eng.fork(op[1], op[2], op[3])
    eng.upload_tables()

    def dev(bits):
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
        return t.view(torch.bfloat16 if c.dtype == "bf16" else torch.float16).cuda()

    # per-layer inputs of the step (the same values every step)
    qs = {l: dev(wl.q_bits(l, 0)) for l in range(c.L)}
    ks = {l: dev(wl.knew_bits(l, 0)) for l in range(c.L)}
    vs = {l: dev(wl.vnew_bits(l, 0)) for l in range(c.L)}
    outs = {l: torch.empty_like(qs[l]) for l in range(c.L)}
    scale = float(wl.scale)

    # The oracle's starting pool: device copies now (before any step writes
    # the pool), moved to host memory only after the timed region -- many GB
    # of freshly touched host memory during timing let the host stall the
    # launch stream.  Every layer when the device has room for the copies.
    snaps_dev = {}
    if opool is not None:
        nl = c.L if args.cpu_layers <= 0 else min(args.cpu_layers, c.L)
        layer_bytes = 2 * eng.pool.nbytes // (2 * c.L)
        free, _ = torch.cuda.mem_get_info()
        nl = max(1, min(nl, int((free - (8 << 30)) // layer_bytes)))
        snap_layers = sorted(set(int(round(i * (c.L - 1) / max(nl - 1, 1))) for i in range(nl)))
        for layer in snap_layers:
            snaps_dev[layer] = tuple(eng.pool.slab(layer, w).clone() for w in ("k", "v"))
    torch.cuda.synchronize()

    # Every timing event exists (and has been recorded once) and the collector
    # has run before the warm-up steps, so that the device idles only for the
    # final synchronisation between warm-up and timing (after an idle spell
    # the first launches run slower).
    hev = HipEvents()
    sh = torch.cuda.current_stream().cuda_stream

    class _Ev:
        def __init__(self):
            self.e = hev.create()
            hev.record(self.e, sh)

        def record(self, stream=None):
            hev.record(self.e, sh if stream is None else stream.cuda_stream)

    step_events = [(_Ev(), _Ev()) for _ in range(K)]
    # one attention call per step is bracketed (a different layer each step):
    # an event record between two kernels costs a few microseconds, so
    # bracketing every call would slow the very step being measured
    attn_pool = [{(7 * i) % c.L: (_Ev(), _Ev())} for i in range(K)]
    ev0, ev1 = _Ev(), _Ev()
    torch.cuda.synchronize()
    attn_events = []
    alg_bytes = 0
    attn_alg = []
    shared = c.length_kind == "lognormal_branches"     # sequences share prompt blocks
    step_tables = []
    import gc
    gc.collect()
    gc.disable()          # no collector pauses inside the timed region
    fork_step = None
    for w in range(W):
        if w == 0:
            # the first step of a workload with shared partial blocks copies
            # them (copy-on-write); it is timed on its own
            f0, f1, f2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            # load the copy kernel before timing it: a pair with src == dst copies nothing
            eng.pool.copy_blocks(torch.zeros((1, 2), dtype=torch.int32, device="cuda"))
            if c.beam:
                eng.reorder(wl.parents(0))
            max_ctx = eng.manager_step()
            torch.cuda.synchronize()
            f0.record()
            npairs = len(eng.last_pairs)
            if npairs:
                eng.pool.copy_blocks(eng.d_pairs[:npairs])
            f1.record()
            eng.device_step(qs, ks, vs, outs, max_ctx, scale, skip_copies=True)
            f2.record()
            torch.cuda.synchronize()
            if npairs:
                tile = eng.pool.nbytes // (2 * c.L * eng.pool.P)
                copy_bytes = npairs * c.L * 2 * tile * 2
                cms = f0.elapsed_time(f1)
                fork_step = {"cow_pairs": npairs, "copy_bytes": int(copy_bytes),
                             "copy_ms": round(cms, 4), "copy_gbs": round(copy_bytes / (cms * 1e-3) / 1e9, 1),
                             "step_ms": round(f0.elapsed_time(f2), 4)}
            continue
        if c.beam:
            eng.reorder(wl.parents(w))
        max_ctx = eng.manager_step()
        eng.device_step(qs, ks, vs, outs, max_ctx, scale)
    torch.cuda.synchronize()

    wall0 = time.perf_counter()
    ev0.record()
    issue_ms = []
    copies = []
    for i in range(K):
        es, ee = step_events[i]
        h0 = time.perf_counter()
        es.record()
        if c.beam:
            eng.reorder(wl.parents(W + i))
        max_ctx = eng.manager_step()
        eng.device_step(qs, ks, vs, outs, max_ctx, scale, attn_events=attn_events,
                        event_pool=attn_pool[i])
        ee.record()
        issue_ms.append((time.perf_counter() - h0) * 1e3)
        ab = attn_bytes(eng.lens, wl.S, c.Hq, c.Hkv, c.d, c.B)
        attn_alg.append(ab)
        if shared:
            step_tables.append((eng.tables.copy(), eng.lens.copy()))
        alg_bytes += c.L * (ab + write_bytes(wl.S, c.Hkv, c.d))
        alg_bytes += len(eng.last_pairs) * c.L * 2 * eng.pool.nbytes // (2 * c.L * wl.P) * 2
        copies.append(len(eng.last_pairs))
    ev1.record()
    torch.cuda.synchronize()
    wall1 = time.perf_counter()
    gc.enable()

    total_ms = hev.elapsed_ms(ev0.e, ev1.e)
    ms_per_step = total_ms / K
    step_ms = np.array([hev.elapsed_ms(a.e, b.e) for a, b in step_events])
    attn_ms = np.array([hev.elapsed_ms(a.e, b.e) for a, b in attn_events])
    hev.close()
    mean_attn_bytes = float(np.mean(attn_alg))
    logical_attn_bytes = mean_attn_bytes
    logical_value = alg_bytes / (total_ms * 1e-3) / 1e9
    if shared:
        # a block that several sequences map is counted once: the bytes the
        # method must move (logical bytes count it once per sequence)
        uniq = np.array([unique_kv_bytes(t, n, c, wl.P) for t, n in step_tables], dtype=np.float64)
        logical_kv = np.array([int(np.sum(n)) * 2 * c.Hkv * c.d * 2 for _, n in step_tables], dtype=np.float64)
        attn_unique = np.array(attn_alg, dtype=np.float64) - logical_kv + uniq
        alg_bytes -= c.L * float(np.sum(logical_kv - uniq))
        mean_attn_bytes = float(np.mean(attn_unique))
    attn_avg_us = float(np.mean(attn_ms)) * 1e3
    achieved = mean_attn_bytes / (attn_avg_us * 1e-6) / 1e9
    value = alg_bytes / (total_ms * 1e-3) / 1e9
    seq_steps = wl.S * K / (total_ms * 1e-3)

    result = {
        "metric": "paged decode-attn achieved HBM GB/s (% of MI355X peak) + seq-steps/sec",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{c.name}: {c.description}; {c.L} layers in sequence, +1 token per step, "
                        f"pool {wl.P} blocks",
            "global_batch": wl.S,
            "layers": c.L,
            "block_size": c.B,
            "shared_prefixes_read_once": bool(grouped),
            "pool_gib": round(eng.pool.nbytes / 2 ** 30, 2),
            "parallelism": "single GPU",
        },
        "seq_steps_per_s": round(seq_steps, 1),
        # internal fragmentation at the last step: used slots / allocated slots
        "slot_utilization": round(float(np.sum(eng.lens)) / float(np.sum(-(-np.asarray(eng.lens) // c.B)) * c.B), 4),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        # the device's time inside the step brackets, and what lies between them
        "gpu_busy_ms_per_step": round(float(np.mean(step_ms)), 4),
        "gap_ms_per_step": round(ms_per_step - float(np.mean(step_ms)), 4),
        "step_ms_p10_p50_p90": [round(float(np.percentile(step_ms, q)), 4) for q in (10, 50, 90)],
        "wall_ms_per_step": round((wall1 - wall0) * 1e3 / K, 4),
        "attn_launch_us_p10_p50_p90": [round(float(np.percentile(attn_ms, q)) * 1e3, 2) for q in (10, 50, 90)],
        "attn_launches_timed": int(len(attn_ms)),
        "roofline": {
            "kernel": (f"grouped: mq_mfma_kernel<{c.dtype},group pass> + decode_attention_kernel<suffix> + "
                       f"cascade merge" if grouped else f"decode_attention_kernel<{c.dtype},G={c.G},B={c.B}> + merge"),
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "traffic_note": "no counter summary for this kernel source",
            "alg_bytes_per_launch": int(mean_attn_bytes),
            "avg_launch_us": round(attn_avg_us, 2),
        },
    }

    if fork_step is not None:
        result["fork_step"] = fork_step
    if c.beam:
        tile = eng.pool.nbytes // (2 * c.L * wl.P)
        live = wl.P - eng.pool.num_free()
        separate = int(np.sum(-(-eng.lens.astype(np.int64) // c.B)))
        result["beam"] = {"width": c.branches, "copies_per_step_mean": round(float(np.mean(copies)), 2),
                          "copy_bytes_per_step_mean": int(np.mean(copies) * c.L * 2 * tile * 2),
                          "live_blocks_last_step": int(live), "blocks_without_sharing": separate,
                          "block_saving": round(1 - live / separate, 4)}
    if shared:
        result["logical_value"] = round(logical_value, 1)
        result["roofline"]["achieved_logical"] = round(logical_attn_bytes / (attn_avg_us * 1e-6) / 1e9, 1)
        result["roofline"]["logical_bytes_per_launch"] = int(logical_attn_bytes)
        result["roofline"]["note"] = ("achieved and value count a block that several sequences map once "
                                      "(unique bytes); the logical figures count it once per sequence, "
                                      "and may exceed the HBM peak since repeated reads hit in cache")
    # counters apply only to the workload and launch mode they were taken on
    here = {"config": args.config, "block_size": c.B, "head_shards": args.head_shards or 1,
            "order": args.order, "grouped": bool(grouped)}
    rec = recorded_traffic(here)
    if rec is not None:
        result["roofline"]["traffic"] = int(rec["traffic_bytes_per_launch"])
        result["roofline"]["traffic_note"] = (
            f"rocprofv3 FETCH_SIZE x{rec['fetch_scale']} + WRITE_SIZE x{rec['write_scale']} per launch "
            f"(scales from a plain copy of known size), at {rec['alg_bytes_per_launch']} algorithmic bytes; "
            f"traffic / algorithmic = {rec['traffic_over_alg']}")
    result["host_issue_ms_per_step_p50"] = round(float(np.median(issue_ms)), 4)
    result["measurement"] = {
        "accumulation": "fp32 (scores, softmax state, weighted values); output rounded to nearest even",
        "inputs": f"Q, K, V ~ N(0,1) rounded to {c.dtype}; seeded per workload, layer and purpose",
        "timing": f"{K} steps after {W} warm-ups, HIP events on the launch stream, inputs resident in HBM",
    }
    result["memory"] = memory_breakdown(eng, wl, c)
    result["stream_ceiling"] = stream_ceiling(eng, c, wl, c.L, achieved=achieved, grouped=bool(grouped))
    if args.dump:
        with open(args.dump, "w") as f:
            json.dump({"step_ms": step_ms.tolist(), "attn_us": (attn_ms * 1e3).tolist(), "issue_ms": issue_ms,
                       "attn_layers": [next(iter(d)) for d in attn_pool]}, f)
    if opool is not None:
        result["cpu_baseline"], result["parity"] = cpu_baseline(wl, eng, snaps_dev, outs, W + K, opool)
    print(json.dumps(result), flush=True)
    return 0


def multi_query_bench(args) -> int:
    """Q new tokens per sequence per step: the host manager reserves their
    slots, pa_write_kv stores their keys/values, and every layer runs
    pa_multi_query_attention (query t of a sequence attends causally up to
    its own position).  Algorithmic bytes per layer: every useful key/value
    position once, the queries and outputs, the tables; flops per layer:
    4 d per (query head, visible position)."""
    import torch

    from paged_kv_cache_239_amd import multi_query_workspace
    from paged_kv_cache_239_amd.engine import DecodeEngine
    from workloads import make_workload, with_headroom

    Q = args.queries
    W = args.warmup if args.warmup is not None else 1
    K = args.steps if args.steps is not None else 6
    wl = with_headroom(make_workload(args.config, block_size=args.block_size or None), (W + K) * Q + 1)
    c = wl.cfg
    maxb = wl.max_blocks((W + K) * Q + 1)
    eng = DecodeEngine(c.L, c.Hq, c.Hkv, c.d, c.B, wl.P, c.dtype, wl.S, maxb, free_order=wl.free_order)
    for layer in range(c.L):
        for which in ("k", "v"):
            g = torch.Generator(device="cuda")
            g.manual_seed(wl.pool_fill_seed(layer, which))
            eng.pool.slab(layer, which).normal_(generator=g)
    for op in wl.history:
        if op[0] == "append":
            eng.append(op[1], op[2])
        else:
            eng.fork(op[1], op[2], op[3])
    T = wl.S * Q
    tdt = torch.bfloat16 if c.dtype == "bf16" else torch.float16
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wl.pool_fill_seed(0, "k") ^ 0x5A5A)
    qs = [torch.randn((T, c.Hq, c.d), generator=gen, device="cuda").to(tdt) for _ in range(c.L)]
    kn = [torch.randn((T, c.Hkv, c.d), generator=gen, device="cuda").to(tdt) for _ in range(c.L)]
    vn = [torch.randn((T, c.Hkv, c.d), generator=gen, device="cuda").to(tdt) for _ in range(c.L)]
    outs = [torch.empty_like(x) for x in qs]
    q_start = torch.arange(0, T + 1, Q, dtype=torch.int32, device="cuda")
    scale = float(wl.scale)
    ws = multi_query_workspace(eng.pool, wl.S, c.Hq, maxb * c.B, Q)
    d_slots = torch.empty(T, dtype=torch.int64, device="cuda")

    def step(events=None):
        slots = np.empty(T, dtype=np.int64)
        pairs = []
        for s in range(wl.S):
            sl, pr = eng.append(s, Q)
            slots[s * Q:(s + 1) * Q] = sl
            pairs += pr
        eng.upload_tables()
        d_slots.copy_(torch.from_numpy(slots))
        if pairs:
            eng.pool.copy_blocks(torch.tensor(pairs, dtype=torch.int32, device="cuda"))
        max_ctx = int(eng.lens.max())
        for layer in range(c.L):
            eng.pool.write_kv(layer, kn[layer], vn[layer], d_slots)
            if events is not None and layer == events[2]:
                events[0].record()
            eng.pool.multi_query_attention(layer, outs[layer], qs[layer], q_start, eng.d_tables, eng.d_lens,
                                           max_ctx, Q, scale, workspace=ws,
                                           host_context_lens=eng.lens if args.order == "on" else None)
            if events is not None and layer == events[2]:
                events[1].record()
        return eng.lens.copy()

    for _ in range(W):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    att = []
    lens_hist = []
    t_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    e0.record()
    for i in range(K):
        lens_hist.append(step((t_ev[i][0], t_ev[i][1], (7 * i) % c.L)))
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    att_us = float(np.mean([a.elapsed_time(b) for a, b in t_ev])) * 1e3

    def layer_bytes(lens):
        lens = np.asarray(lens, dtype=np.int64)
        return (int(lens.sum()) * 2 * c.Hkv * c.d * 2 + 2 * T * c.Hq * c.d * 2
                + int(np.sum(-(-lens // c.B))) * 4 + wl.S * 8)

    def layer_flops(lens):
        # query t of nq sees n - nq + t + 1 positions; 4 d flops per (head, position)
        vis = sum(int(n) * Q - Q * (Q - 1) // 2 for n in lens)
        return 4 * c.d * c.Hq * vis

    ab = float(np.mean([layer_bytes(x) for x in lens_hist]))
    fl = float(np.mean([layer_flops(x) for x in lens_hist]))
    wbytes = 2 * (2 * T * c.Hkv * c.d * 2) + 8 * T
    step_bytes = c.L * (ab + wbytes)
    gbs = ab / (att_us * 1e-6) / 1e9
    tfs = fl / (att_us * 1e-6) / 1e12
    # more than 8 rows (query tokens x heads) per sequence run on the matrix
    # cores (dense 16-bit MFMA peak), fewer on the fp32 vector units
    mfma = Q * c.G > 8
    cpeak = 2500.0 if mfma else 157.3
    ridge = cpeak * 1e12 / (HBM_PEAK_GBS * 1e9)          # flop per byte where the roofs meet
    mem_bound = fl / ab < ridge
    hbm = gbs / HBM_PEAK_GBS
    alu = tfs / cpeak
    res = {
        "metric": "multi-query paged attention: achieved HBM GB/s and TFLOP/s + query tokens/s",
        "value": round(step_bytes / (ms * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "dtype": c.dtype, "data": "synthetic",
        "config": {"workload": f"{c.name}: every step appends {Q} tokens to each of {wl.S} sequences "
                               f"(context {int(wl.lengths0.min()) - 1}..{int(wl.lengths0.max()) - 1} before the first step)",
                   "queries_per_sequence": Q, "block_size": c.B, "layers": c.L},
        "query_tokens_per_s": round(T / (ms * 1e-3), 1),
        "roofline": {"kernel": (f"mq_wide_kernel<{c.dtype},G={c.G},B={c.B}> (whole context per workgroup, no merge)"
                                if Q * c.G > 32 else
                                f"mq_mfma_kernel<{c.dtype},G={c.G},B={c.B}> + merge" if mfma else
                                f"decode_attention_kernel<{c.dtype},rows=8,B={c.B},QT={8 // c.G}> + merge"),
                     "bound": "hbm" if mem_bound else ("mfma" if mfma else "alu"),
                     "achieved": round(gbs, 1) if mem_bound else round(tfs, 2),
                     "peak": HBM_PEAK_GBS if mem_bound else cpeak,
                     "unit": "GB/s" if mem_bound else "TFLOP/s",
                     "frac": round(hbm if mem_bound else alu, 4),
                     "hbm_gbs": round(gbs, 1), "tflops": round(tfs, 2),
                     "compute_peak_tflops": cpeak,
                     "intensity_flop_per_byte": round(fl / ab, 1), "ridge_flop_per_byte": round(ridge, 1),
                     "alg_bytes_per_launch": int(ab), "flops_per_launch": int(fl),
                     "avg_launch_us": round(att_us, 2),
                     "note": "bound from the arithmetic intensity of the algorithmic bytes and flops against "
                             "the ridge point; compute peak: dense 16-bit MFMA 2.5 PFLOP/s on the matrix path, "
                             "fp32 vector 157.3 TFLOP/s on the vector path",
                     "traffic": None},
    }
    rec = recorded_traffic({"config": args.config, "block_size": c.B, "queries": Q, "order": args.order})
    if rec is not None:
        res["roofline"]["traffic"] = int(rec["traffic_bytes_per_launch"])
        res["roofline"]["traffic_note"] = (
            f"rocprofv3 FETCH_SIZE x{rec['fetch_scale']} + WRITE_SIZE x{rec['write_scale']} per call, at "
            f"{rec['alg_bytes_per_launch']} algorithmic bytes; traffic / algorithmic = {rec['traffic_over_alg']}")
    print(json.dumps(res), flush=True)
    return 0


def swap_bench(args) -> int:
    """Preemption by swapping: the first N sequences of the workload (all
    their blocks, every layer) move to a pinned host pool and back, each
    direction one pa_swap_blocks launch in which the GPU writes or reads host
    memory directly.  For comparison a sample of the same tiles is copied
    with one DMA transfer per tile (per layer, keys and values: the many
    short transfers that small blocks turn a swap into).  Bytes = moved
    blocks x 2 L tiles; the round trip is checked byte for byte."""
    import torch

    from paged_kv_cache_239_amd import Pool
    from paged_kv_cache_239_amd.engine import DecodeEngine
    from workloads import make_workload

    wl = make_workload(args.config, block_size=args.block_size or None)
    c = wl.cfg
    eng = DecodeEngine(c.L, c.Hq, c.Hkv, c.d, c.B, wl.P, c.dtype, wl.S, wl.max_blocks(1), free_order=wl.free_order)
    for layer in range(c.L):
        for which in ("k", "v"):
            g = torch.Generator(device="cuda")
            g.manual_seed(wl.pool_fill_seed(layer, which))
            eng.pool.slab(layer, which).normal_(generator=g)
    for op in wl.history:
        if op[0] == "append":
            eng.append(op[1], op[2])
        else:
            eng.fork(op[1], op[2], op[3])
    N = min(args.swap, wl.S)
    group = eng.tables[:N].copy()
    lens = eng.lens[:N].copy()
    need = len(np.unique(np.concatenate([group[s, : -(-int(n) // c.B)] for s, n in enumerate(lens)])))
    host = Pool(c.L, c.Hkv, c.d, c.B, need, c.dtype, device="pinned")
    dev = eng.pool
    tile = dev.nbytes // (2 * c.L * wl.P)
    slab_d, slab_h = wl.P * tile, need * tile

    def tiles_of(pool_buf, slab, blocks):
        # [2L][n][tile] view of the given blocks of every slab
        idx = torch.as_tensor(np.asarray(blocks, dtype=np.int64), device=pool_buf.device)
        v = pool_buf.view(2 * c.L, slab // tile, tile)
        return v.index_select(1, idx)

    torch.cuda.synchronize()
    # load the kernel before timing (a pair outside both pools copies nothing)
    dev.swap_blocks(host, torch.tensor([[wl.P, need]], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    t0 = time.perf_counter()
    pairs = dev.move_blocks(host, group, lens)
    t1 = time.perf_counter()
    before = tiles_of(dev.buffer, slab_d, pairs[:, 0]).clone()
    d_pairs = torch.from_numpy(pairs).cuda()
    torch.cuda.synchronize()
    e[0].record()
    dev.swap_blocks(host, d_pairs)
    e[1].record()
    torch.cuda.synchronize()
    # the device blocks are free now: overwrite them, as the next user would
    dv = dev.buffer.view(2 * c.L, wl.P, tile)
    dv.index_fill_(1, torch.as_tensor(pairs[:, 0].astype(np.int64), device="cuda"), 0)
    t2 = time.perf_counter()
    back = host.move_blocks(dev, group, lens)
    t3 = time.perf_counter()
    d_back = torch.from_numpy(back).cuda()
    torch.cuda.synchronize()
    e[2].record()
    host.swap_blocks(dev, d_back)
    e[3].record()
    torch.cuda.synchronize()
    # back[i] = (host block, new device block) in the order pairs[i] = (old device block, host block)
    order = {int(h): i for i, h in enumerate(pairs[:, 1])}
    perm = np.array([order[int(h)] for h in back[:, 0]])
    after = tiles_of(dev.buffer, slab_d, back[:, 1])
    exact = bool(torch.equal(after, before[:, perm]))
    nbytes = len(pairs) * 2 * c.L * tile
    out_ms, in_ms = e[0].elapsed_time(e[1]), e[2].elapsed_time(e[3])
    # per-tile DMA copies, on a sample of the blocks (device -> host)
    sample = min(len(pairs), max(1, 4096 // (2 * c.L)))
    dsrc = dev.buffer.view(2 * c.L, wl.P, tile)
    hdst = host.buffer.view(2 * c.L, need, tile)
    torch.cuda.synchronize()
    e[4].record()
    for i in range(sample):
        a, b = int(back[i, 1]), int(back[i, 0])
        for sl in range(2 * c.L):
            hdst[sl, b].copy_(dsrc[sl, a], non_blocking=True)
    e[5].record()
    torch.cuda.synchronize()
    dma_ms = e[4].elapsed_time(e[5])
    dma_bytes = sample * 2 * c.L * tile
    res = {
        "metric": "swap GB/s: device pool <-> pinned host pool, one kernel launch per direction",
        "value": round(nbytes / (out_ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "higher_is_better": True,
        "dtype": c.dtype,
        "data": "synthetic",
        "config": {"workload": f"{c.name}: first {N} sequences ({int(lens.sum())} tokens), all {c.L} layers",
                   "block_size": c.B, "tile_bytes": int(tile), "blocks": int(len(pairs)), "bytes": int(nbytes)},
        "swap_out_ms": round(out_ms, 3),
        "swap_in_ms": round(in_ms, 3),
        "swap_in_gbs": round(nbytes / (in_ms * 1e-3) / 1e9, 2),
        "host_manager_ms": {"out": round((t1 - t0) * 1e3, 3), "in": round((t3 - t2) * 1e3, 3)},
        "per_tile_dma": {"tiles": sample * 2 * c.L, "tile_bytes": int(tile), "ms": round(dma_ms, 3),
                         "gbs": round(dma_bytes / (dma_ms * 1e-3) / 1e9, 2),
                         "note": "one hipMemcpyAsync per (block, layer, keys or values) tile, device to host"},
        "round_trip_bit_exact": exact,
    }
    print(json.dumps(res), flush=True)
    return 0 if exact else 1


def memory_breakdown(eng, wl, c) -> dict:
    """Where the pool's and the step's device memory goes at the end of the
    run ("PagedAttention and Online Inference", section 6: useful key/value
    state, tail-block fragmentation, block tables, workspaces and reserved
    pools, counted apart).  A physical block that several sequences map is
    counted once, with the most positions any of them uses."""
    per_pos = 2 * c.L * c.Hkv * c.d * 2                 # keys and values of one slot, every layer
    st = eng.pool.stats()
    lens = eng.lens.astype(np.int64)
    nb = -(-lens // c.B)
    used = np.zeros(wl.P, dtype=np.int64)
    for s in range(wl.S):
        for j in range(int(nb[s])):
            b = int(eng.tables[s, j])
            used[b] = max(used[b], min(c.B, int(lens[s]) - j * c.B))
    live = int(np.count_nonzero(used))
    useful = int(used.sum())
    ws = int(eng.ws_bytes) + int(eng.gws_bytes)
    return {
        "pool_bytes": int(eng.pool.nbytes),
        "useful_kv_bytes": useful * per_pos,
        "tail_slot_bytes": (live * c.B - useful) * per_pos,
        "free_block_bytes": int(st["free_blocks"]) * c.B * per_pos,
        "block_table_bytes": int(eng.d_tables.numel()) * 4,
        "lengths_slots_pairs_bytes": int(eng.d_lens.numel()) * 4 + int(eng.d_slots.numel()) * 8
                                     + int(eng.d_pairs.numel()) * 4,
        "workspace_bytes": ws,
        "useful_fraction_of_pool": round(useful * per_pos / eng.pool.nbytes, 4),
        "useful_fraction_of_live_blocks": round(useful / max(live * c.B, 1), 4),
        "manager": {"allocs": int(st["allocs"]), "cows": int(st["cows"]), "releases": int(st["releases"]),
                    "live_blocks": int(st["live_blocks"]), "live_high_water": int(st["live_high_water"]),
                    "free_blocks": int(st["free_blocks"]), "num_blocks": int(st["num_blocks"])},
    }


def stream_ceiling(eng, c, wl, layers, achieved, grouped) -> dict:
    """Achievable read rate for the attention's own access pattern:
    pa_stream_tiles reads exactly the key/value rows of the final step
    (through the real, shuffled block tables, then through tables that
    place every sequence's blocks consecutively), one launch per layer, timed
    with HIP events around all of them."""
    import torch
    lens = eng.lens.astype(np.int64)
    kv = int(lens.sum()) * 2 * c.Hkv * c.d * 2
    nb = -(-lens // c.B)
    seq_tables = np.zeros_like(eng.tables)
    start = 0
    for s in range(wl.S):
        seq_tables[s, : nb[s]] = np.arange(start, start + nb[s])
        start += int(nb[s])
    out = {"kernel": f"stream_tiles_kernel<B={c.B}>", "kv_bytes_per_launch": kv, "launches": layers}
    chk = torch.zeros(1, dtype=torch.int32, device="cuda")
    max_ctx = int(lens.max())
    for name, tabs in (("shuffled_tables", eng.d_tables), ("consecutive_blocks", torch.from_numpy(seq_tables).cuda())):
        for _ in range(2):      # load the kernel, then time
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for l in range(layers):
                eng.pool.stream_tiles(l, tabs, eng.d_lens, max_ctx, chk)
            e1.record()
            torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / layers
        out[name] = {"us_per_launch": round(us, 2), "gbs": round(kv / (us * 1e-6) / 1e9, 1)}
    ceil = out["shuffled_tables"]["gbs"]
    if not grouped:
        out["attention_frac_of_ceiling"] = round(achieved / ceil, 4)
    out["ceiling_frac_of_peak"] = round(ceil / HBM_PEAK_GBS, 4)
    return out


def cpu_baseline(wl, eng, snaps_dev, outs, total_steps, opool):
    """The fp64 oracle on the final timed step, every snapshotted layer x
    every sequence, over a process pool on the host's cores.  Its own
    manager replays the history and every step; its own copy of each layer
    (the device snapshot taken before any step, i.e. torch's seeded fill)
    receives every step's copies and writes; then the layer's sequences are
    decoded in parallel.  Timed: the parallel decode (gather + dense
    attention) of every (layer, sequence)."""
    import torch

    from oracle.cache_ops import HostPool, copy_blocks, write_kv
    from oracle.dtypes import bits_to_f64
    from oracle.replay import beam_reorder, build_state, manager_step
    from tests.harness import ATOL, RTOL, tol_stats

    c = wl.cfg
    st = build_state(wl, maxb=eng.maxb)
    history = []
    for step in range(total_steps):
        if c.beam:
            beam_reorder(st, wl.parents(step))
        slots, pairs, lens = manager_step(st)
        history.append((list(slots), list(pairs)))
    tables_match = bool(np.array_equal(np.asarray(st.lens), eng.lens)) and all(
        list(eng.tables[s, : -(-st.lens[s] // c.B)]) == st.tables[s][: -(-st.lens[s] // c.B)]
        for s in range(wl.S))

    secs = busy = 0.0
    nbytes, done = 0, 0
    worst = {"max_abs": 0.0, "abs_margin_worst": -1.0, "max_rel": 0.0, "allclose_worst": -1.0}
    finite = True
    layers_done = []
    for l in sorted(snaps_dev):
        kd, vd = snaps_dev.pop(l)
        K, V = opool.layer_buffer(tuple(kd.shape))
        torch.from_numpy(K.view(np.int16)).copy_(kd.view(torch.int16).cpu())
        torch.from_numpy(V.view(np.int16)).copy_(vd.view(torch.int16).cpu())
        del kd, vd
        pool = HostPool.from_arrays(K[None], V[None])
        for slots, pairs in history:
            copy_blocks(pool, pairs)
            write_kv(pool, 0, wl.knew_bits(l, 0), wl.vnew_bits(l, 0), slots)
        ref, wall, b = opool.decode_layer(wl.q_bits(l, 0), st.tables, st.lens, float(wl.scale), c.dtype)
        secs += wall
        busy += b
        got = bits_to_f64(outs[l].view(torch.int16).cpu().numpy().view(np.uint16), c.dtype)
        ts = tol_stats(got, ref, c.dtype)
        finite = finite and ts["finite"]
        for k in worst:
            worst[k] = max(worst[k], ts[k])
        nbytes += attn_bytes(st.lens, wl.S, c.Hq, c.Hkv, c.d, c.B)
        done += wl.S
        layers_done.append(l)
    all_layers = len(layers_done) == c.L
    baseline = {
        "value": round(nbytes / secs / 1e9, 4),
        "unit": "GB/s",
        "cores": opool.workers,
        "kind": "oracle",
        "seq_steps_per_s": round(done / c.L / secs, 3),
        "seconds": round(secs, 2),
        "worker_busy_seconds": round(busy, 2),
        "sample": (f"final timed step, {'all ' if all_layers else ''}{len(layers_done)} of {c.L} layers x all "
                   f"{wl.S} sequences ({done} sequence-layers); numpy fp64 gather + dense attention, "
                   f"{opool.workers} worker processes with one BLAS thread each"
                   + ("" if all_layers else f"; layers {layers_done}, seq-steps/s scaled by 1/{c.L} layers")),
    }
    ok = finite and worst["abs_margin_worst"] <= 0.0 and worst["max_rel"] <= RTOL and tables_match
    parity = {"seq_layers_checked": done, "of": wl.S * c.L,
              "max_abs": worst["max_abs"], "abs_margin_worst": worst["abs_margin_worst"],
              "max_rel_where_ref_at_least_0.2": worst["max_rel"], "allclose_worst": worst["allclose_worst"],
              "tolerance": {"rule": ("every element |o-r| <= 2e-3" if c.dtype == "f16" else
                                     "every element |o-r| <= 2e-3 + half a bf16 ulp of max(|o|,|r|) (the "
                                     "output's own rounding)") + "; |o-r|/|r| <= 1e-2 where |r| >= 0.2",
                            "max_abs": ATOL, "max_rel": RTOL},
              "pass": bool(ok), "tables_bit_exact": tables_match}
    return baseline, parity


if __name__ == "__main__":
    sys.exit(main())
