"""One decode step over a paged pool, end to end.

Per step (batch of S sequences, each appending one token):
  1. host manager (libpa): every sequence reserves the slot of its new token,
     in batch order; writes into shared partial blocks request a
     copy-on-write pair ("vLLM PagedAttention and continuous batching",
     sections "PagedAttention: fixed blocks, non-contiguous physical memory"
     and "Sharing with reference counts and copy-on-write");
  2. upload of block tables, context lengths, slots and copy pairs (pinned
     staging buffers, asynchronous on the stream);
  3. pa_copy_blocks for the copy-on-write pairs, before any write;
  4. for every layer: the new token's cache write and the attention, in one
     pass (pa_write_kv_decode_attention) or as pa_write_kv then
     pa_decode_attention.  With ``grouped``, sequences that share leading
     blocks (parallel samples, beams) are found after the appends
     (pa_prefix_groups) and their shared positions are read once per group
     (pa_decode_attention_grouped).

Everything in steps 1, 3 and 4 runs in the native library; this module only
sequences the calls and moves arguments.
"""

from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np

from ._abi import check
from .pool import Pool, _ptr, _stream_handle


class _Staging:
    """Ring of pinned host buffers guarded by events, so the host can run
    several steps ahead of the device without overwriting a buffer that an
    earlier asynchronous copy still reads.

    The wait for a buffer polls its event: a blocking wait may wake the host
    milliseconds after the event completes, and with only a few steps queued
    the device then runs dry (one step in twenty took 8.5 ms instead of
    3.2 ms).  Eight buffers keep about eight steps of work queued."""

    def __init__(self, nbytes: int, depth: int = 8):
        import torch
        self.bufs = [torch.empty(nbytes, dtype=torch.uint8, pin_memory=True) for _ in range(depth)]
        self.events = [torch.cuda.Event() for _ in range(depth)]
        self.armed = [False] * depth
        self.i = 0

    def next(self):
        j = self.i
        self.i = (self.i + 1) % len(self.bufs)
        if self.armed[j]:
            ev = self.events[j]
            while not ev.query():
                pass
        return j, self.bufs[j]

    def mark(self, j, stream):
        self.events[j].record(stream)
        self.armed[j] = True


class DecodeEngine:
    def __init__(self, L: int, Hq: int, Hkv: int, d: int, B: int, P: int, dtype: str, S: int, maxb: int,
                 free_order: Optional[Sequence[int]] = None, device: str = "cuda", fused: bool = True,
                 grouped: bool = False, ordered: bool = True, debug: bool = False):
        import torch
        self.torch = torch
        self.fused = fused
        # check every step's tables, lengths and slots against the manager
        # (pa_validate_step) before they are uploaded
        self.debug = debug
        # launch the context partitions longest first from the manager's own
        # lengths (pa_decode_attention_ordered)
        self.ordered = ordered
        self.grouped = grouped
        self.L, self.Hq, self.Hkv, self.d, self.B, self.P = L, Hq, Hkv, d, B, P
        self.S, self.maxb = S, maxb
        self.device = device
        self.pool = Pool(L, Hkv, d, B, P, dtype, free_order=free_order, device=device)
        self.tables = np.full((S, maxb), -1, dtype=np.int32)   # host block tables
        self.lens = np.zeros(S, dtype=np.int32)                 # tokens held per sequence
        self.d_tables = torch.zeros((S, maxb), dtype=torch.int32, device=device)
        self.d_lens = torch.zeros(S, dtype=torch.int32, device=device)
        self.d_slots = torch.zeros(S, dtype=torch.int64, device=device)
        self.d_pairs = torch.zeros((S, 2), dtype=torch.int32, device=device)
        # shared-prefix runs of the current step (grouped mode)
        self.d_group_start = torch.zeros(S + 1, dtype=torch.int32, device=device)
        self.d_group_len = torch.zeros(S, dtype=torch.int32, device=device)
        self.d_seq_group = torch.zeros(S, dtype=torch.int32, device=device)
        self.n_groups = self.max_group = self.max_shared = self.max_suffix = 0
        self.host_group_len = np.zeros(0, dtype=np.int32)
        self.gws = None
        self.gws_bytes = 0
        self._gcap = 0
        self._stage_bytes = S * maxb * 4 + S * 4 + S * 8 + S * 8 + (3 * S + 1) * 4
        self._staging = _Staging(self._stage_bytes)
        self.ws = None
        self.ws_bytes = 0
        self.last_pairs = np.zeros((0, 2), dtype=np.int32)
        self.last_slots = np.zeros(0, dtype=np.int64)

    # ---- history (prefill / sharing) ----------------------------------------------
    def append(self, s: int, ntok: int):
        """Prefill ``ntok`` tokens onto sequence s: returns (slots, cow pairs)."""
        slots, pairs = self.pool.append_tokens(self.tables[s], int(self.lens[s]), ntok)
        self.lens[s] += ntok
        return slots, pairs

    def fork(self, child: int, parent: int, ntok: int) -> None:
        self.pool.fork(self.tables[parent], ntok, self.tables[child])
        self.lens[child] = ntok

    def reorder(self, parents) -> None:
        """Beam selection before a step: sequence i continues old sequence
        parents[i]; the old tables are released (pa_seq_reorder)."""
        tables, lens = self.pool.seq_reorder(self.tables, self.lens, parents)
        self.tables[:] = tables
        self.lens[:] = lens

    def upload_tables(self, stream=None) -> None:
        """Synchronous upload of the current tables and lengths."""
        torch = self.torch
        self.d_tables.copy_(torch.from_numpy(self.tables))
        self.d_lens.copy_(torch.from_numpy(self.lens))

    # ---- workspace ------------------------------------------------------------------
    def ensure_workspace(self, max_ctx: int, stream=None) -> None:
        # sized once for the longest context the tables can hold
        need = self.pool.workspace_bytes(self.S, self.Hq, max(max_ctx, self.maxb * self.B))
        if need > self.ws_bytes:
            torch = self.torch
            self.ws = torch.empty(need, dtype=torch.uint8, device=self.device)
            check(self.pool.lib, self.pool.lib.pa_decode_workspace_init(_ptr(self.ws), need,
                                                                        _stream_handle(stream)))
            self.ws_bytes = need

    # ---- one decode step ----------------------------------------------------------------
    def manager_step(self, stream=None) -> int:
        """Host manager for one step plus the asynchronous upload of its
        results.  Returns the step's max context length."""
        torch = self.torch
        n_before = self.lens.copy()
        slots, pairs = self.pool.append_batch(self.tables, n_before)
        self.lens += 1
        self.last_slots, self.last_pairs = slots, pairs
        if self.debug:
            self.pool.validate_step(self.tables, self.lens, slots)
        S, mb = self.S, self.maxb
        if self.grouped:
            gs, gl, sg, self.max_group, self.max_shared, self.max_suffix = self.pool.prefix_groups(self.tables,
                                                                                                   self.lens)
            self.n_groups = len(gl)
            self.host_group_len = gl
        j, buf = self._staging.next()
        o = 0
        tb = buf[o:o + S * mb * 4]; o += S * mb * 4
        lb = buf[o:o + S * 4]; o += S * 4
        sb = buf[o:o + S * 8]; o += S * 8
        pb = buf[o:o + S * 8]; o += S * 8
        gb = buf[o:o + (3 * S + 1) * 4]
        tb.numpy().view(np.int32)[:] = self.tables.reshape(-1)
        lb.numpy().view(np.int32)[:] = self.lens
        sb.numpy().view(np.int64)[:] = slots
        npairs = len(pairs)
        if npairs:
            pb.numpy().view(np.int32)[: 2 * npairs] = pairs.reshape(-1)
        st = torch.cuda.current_stream() if stream is None else stream
        if self.grouped:
            g = gb.numpy().view(np.int32)
            ng = self.n_groups
            g[: ng + 1] = gs
            g[S + 1: S + 1 + ng] = gl
            g[2 * S + 1: 3 * S + 1] = sg
        with torch.cuda.stream(st):
            self.d_tables.view(-1).view(torch.uint8).copy_(tb, non_blocking=True)
            self.d_lens.view(torch.uint8).copy_(lb, non_blocking=True)
            self.d_slots.view(torch.uint8).copy_(sb, non_blocking=True)
            if npairs:
                self.d_pairs[:npairs].view(-1).view(torch.uint8).copy_(pb[: 8 * npairs], non_blocking=True)
            if self.grouped:
                gi = gb.view(torch.int32)
                self.d_group_start.copy_(gi[: S + 1], non_blocking=True)
                self.d_group_len.copy_(gi[S + 1: 2 * S + 1], non_blocking=True)
                self.d_seq_group.copy_(gi[2 * S + 1: 3 * S + 1], non_blocking=True)
        self._staging.mark(j, st)
        return int(self.lens.max())

    def ensure_grouped_workspace(self, stream=None) -> None:
        # sized for any run count, shared length up to the table width, and
        # runs up to the next power of two above the largest one so far
        cap = max(2, 1 << (max(self.max_group, 1) - 1).bit_length())
        if cap <= self._gcap and self.gws is not None:
            return
        full = self.maxb * self.B
        need = self.pool.grouped_workspace_bytes(self.S, self.Hq, full, self.S, min(cap, self.S), full, full)
        torch = self.torch
        self.gws = torch.empty(need, dtype=torch.uint8, device=self.device)
        check(self.pool.lib, self.pool.lib.pa_decode_workspace_init(_ptr(self.gws), need, _stream_handle(stream)))
        self.gws_bytes = need
        self._gcap = cap

    def device_step(self, qs: List, knews: List, vnews: List, outs: List, max_ctx: int, scale: float,
                    stream=None, layers: Optional[Sequence[int]] = None, attn_events=None,
                    event_pool=None, skip_copies: bool = False) -> None:
        """Copies for this step's copy-on-write pairs, then per layer the
        new token's write and the attention.  qs/knews/vnews/outs are indexed
        by layer.  ``attn_events``, if given, is a list that receives one
        (start, end) pair of recorded events around the attention launches of
        the layers in ``event_pool`` (a dict layer -> (start, end) event
        pair); without a pool every layer gets a fresh pair."""
        npairs = len(self.last_pairs)
        if npairs and not skip_copies:
            self.pool.copy_blocks(self.d_pairs[:npairs], stream=stream)
        self.ensure_workspace(max_ctx, stream)
        grouped = self.grouped and self.max_shared > 0
        if grouped:
            self.ensure_grouped_workspace(stream)
        torch = self.torch
        st = None
        if attn_events is not None:
            st = torch.cuda.current_stream() if stream is None else stream
        for layer in (range(self.L) if layers is None else layers):
            if not self.fused:
                self.pool.write_kv(layer, knews[layer], vnews[layer], self.d_slots, stream=stream)
            timed = st is not None and (event_pool is None or layer in event_pool)
            if timed:
                if event_pool is not None:
                    e0, e1 = event_pool[layer]
                else:
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(st)
            if grouped:
                fused = self.fused
                self.pool.decode_attention_grouped(
                    layer, outs[layer], qs[layer], self.d_tables, self.d_lens, max_ctx,
                    self.d_group_start[: self.n_groups + 1], self.d_group_len[: self.n_groups], self.d_seq_group,
                    self.max_group, self.max_shared, self.max_suffix, scale, self.gws,
                    k=knews[layer] if fused else None, v=vnews[layer] if fused else None,
                    slot_mapping=self.d_slots if fused else None, stream=stream,
                    host_group_len=self.host_group_len if self.ordered else None)
            elif self.ordered:
                fused = self.fused
                self.pool.decode_attention_ordered(
                    layer, outs[layer], qs[layer], self.d_tables, self.d_lens, self.lens, max_ctx, scale,
                    workspace=self.ws, k=knews[layer] if fused else None, v=vnews[layer] if fused else None,
                    slot_mapping=self.d_slots if fused else None, stream=stream)
            elif self.fused:
                self.pool.write_kv_decode_attention(layer, knews[layer], vnews[layer], self.d_slots, outs[layer],
                                                    qs[layer], self.d_tables, self.d_lens, max_ctx, scale,
                                                    workspace=self.ws, stream=stream)
            else:
                self.pool.decode_attention(layer, outs[layer], qs[layer], self.d_tables, self.d_lens, max_ctx,
                                           scale, workspace=self.ws, stream=stream)
            if timed:
                e1.record(st)
                attn_events.append((e0, e1))

    def step(self, qs, knews, vnews, outs, scale: float, stream=None) -> None:
        max_ctx = self.manager_step(stream)
        self.device_step(qs, knews, vnews, outs, max_ctx, scale, stream)
