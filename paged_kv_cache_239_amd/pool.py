"""Pool object: host manager calls and device operations of libpa.so."""

from __future__ import annotations

import ctypes as C
from typing import List, Optional, Sequence, Tuple

import numpy as np

from . import _abi
from ._abi import PA_BF16, PA_F16, check, pa_pool_stats

_DTYPES = {"f16": PA_F16, "fp16": PA_F16, "float16": PA_F16, "bf16": PA_BF16, "bfloat16": PA_BF16}


def dtype_code(dtype) -> int:
    if isinstance(dtype, int):
        return dtype
    name = str(dtype).replace("torch.", "")
    return _DTYPES[name]


def _i32p(a: np.ndarray):
    return a.ctypes.data_as(C.POINTER(C.c_int32))


def _i64p(a: np.ndarray):
    return a.ctypes.data_as(C.POINTER(C.c_int64))


def _as_i32(a) -> np.ndarray:
    arr = np.ascontiguousarray(a, dtype=np.int32)
    return arr


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t) -> int:
    return int(t.data_ptr())


class Pool:
    """A paged K/V pool: L layers x (K, V) slabs of P blocks [P][Hkv][B][d].

    ``device`` given: the pool's memory is a torch uint8 tensor owned by this
    object, on that device, or in pinned host memory for ``device="pinned"``
    (a swap pool).  ``device=None`` builds a manager-only pool (no memory;
    device operations are unavailable), used by host-side tests.
    """

    def __init__(self, L: int, Hkv: int, d: int, B: int, P: int, dtype="f16",
                 free_order: Optional[Sequence[int]] = None, device: Optional[str] = "cuda",
                 host_only_lib: bool = False):
        self.lib = _abi.load(host_only=host_only_lib)
        self.L, self.Hkv, self.d, self.B, self.P = L, Hkv, d, B, P
        self.dtype = dtype_code(dtype)
        self.nbytes = int(self.lib.pa_pool_bytes(L, Hkv, d, B, P, self.dtype))
        if self.nbytes == 0:
            raise _abi.PAError(_abi.PA_ERR_INVALID_ARG, "pa_pool_bytes returned 0 for these sizes")
        self.buffer = None
        if device == "pinned":
            # pinned host memory, mapped into the device's address space: a
            # swap target for pa_swap_blocks
            import torch
            self.buffer = torch.empty(self.nbytes, dtype=torch.uint8, pin_memory=True)
            base, nbytes = _ptr(self.buffer), self.nbytes
        elif device is not None:
            import torch
            if str(device) == "cpu":
                # plain host memory carries no alignment promise: over-allocate
                raw = torch.empty(self.nbytes + 256, dtype=torch.uint8)
                off = (-_ptr(raw)) % 256
                self.buffer = raw[off: off + self.nbytes]
            else:
                self.buffer = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
            base, nbytes = _ptr(self.buffer), self.nbytes
        else:
            base, nbytes = 256, self.nbytes   # stand-in address, never dereferenced
        order = None
        if free_order is not None:
            self._order = _as_i32(free_order)
            order = _i32p(self._order)
        handle = C.c_void_p()
        check(self.lib, self.lib.pa_alloc_pool(C.byref(handle), L, Hkv, d, B, P, self.dtype,
                                               C.c_void_p(base), C.c_size_t(nbytes), order))
        self.handle = handle

    def close(self):
        if getattr(self, "handle", None):
            self.lib.pa_free_pool(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---- device views ---------------------------------------------------------
    @property
    def torch_dtype(self):
        import torch
        return torch.bfloat16 if self.dtype == PA_BF16 else torch.float16

    def slab(self, layer: int, which: str):
        """Torch view [P][Hkv][B][d] of one layer's key ("k") or value ("v") slab."""
        if self.buffer is None:
            raise RuntimeError("manager-only pool has no device memory")
        k = C.c_void_p()
        v = C.c_void_p()
        check(self.lib, self.lib.pa_pool_layer_ptrs(self.handle, layer, C.byref(k), C.byref(v)))
        addr = (k.value if which == "k" else v.value) or 0
        off = addr - _ptr(self.buffer)
        slab_bytes = self.P * self.Hkv * self.B * self.d * 2
        return self.buffer[off: off + slab_bytes].view(self.torch_dtype).view(self.P, self.Hkv, self.B, self.d)

    # ---- host manager -----------------------------------------------------------
    def alloc(self) -> int:
        b = C.c_int32()
        check(self.lib, self.lib.pa_block_alloc(self.handle, C.byref(b)))
        return b.value

    def incref(self, blk: int) -> None:
        check(self.lib, self.lib.pa_block_incref(self.handle, int(blk)))

    def decref(self, blk: int) -> None:
        check(self.lib, self.lib.pa_block_decref(self.handle, int(blk)))

    def refcount(self, blk: int) -> int:
        return int(self.lib.pa_block_refcount(self.handle, int(blk)))

    def refcounts(self) -> List[int]:
        return [self.refcount(b) for b in range(self.P)]

    def num_free(self) -> int:
        return int(self.lib.pa_num_free_blocks(self.handle))

    def free_list(self) -> List[int]:
        out = np.zeros(self.P, dtype=np.int32)
        cnt = C.c_int32()
        check(self.lib, self.lib.pa_free_list(self.handle, _i32p(out), self.P, C.byref(cnt)))
        return out[: cnt.value].tolist()

    def stats(self) -> dict:
        st = pa_pool_stats()
        check(self.lib, self.lib.pa_pool_get_stats(self.handle, C.byref(st)))
        return {f: getattr(st, f) for f, _ in st._fields_}

    def append_slot(self, table: np.ndarray, n_before: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        """``table``: int32 numpy array, edited in place."""
        assert table.dtype == np.int32 and table.flags.c_contiguous
        slot = C.c_int64()
        src = C.c_int32()
        dst = C.c_int32()
        check(self.lib, self.lib.pa_append_slot(self.handle, _i32p(table), table.shape[-1], int(n_before),
                                                C.byref(slot), C.byref(src), C.byref(dst)))
        return slot.value, ((src.value, dst.value) if src.value >= 0 else None)

    def append_tokens(self, table: np.ndarray, n_before: int, count: int):
        assert table.dtype == np.int32 and table.flags.c_contiguous
        slots = np.zeros(max(count, 1), dtype=np.int64)
        pairs = np.zeros((max(count, 1), 2), dtype=np.int32)
        npairs = C.c_int32()
        ndone = C.c_int32()
        st = self.lib.pa_append_tokens(self.handle, _i32p(table), table.shape[-1], int(n_before), int(count),
                                       _i64p(slots), _i32p(pairs), C.byref(npairs), C.byref(ndone))
        check(self.lib, st, ndone.value)
        return slots[:count], [tuple(p) for p in pairs[: npairs.value].tolist()]

    def append_batch(self, tables: np.ndarray, n_before: np.ndarray):
        """One decode step.  tables: int32 [S][maxb] (edited in place);
        n_before: int32 [S].  Returns (slots int64 [S], pairs int32 [N][2])."""
        assert tables.dtype == np.int32 and tables.flags.c_contiguous and tables.ndim == 2
        nb = _as_i32(n_before)
        S, maxb = tables.shape
        slots = np.zeros(max(S, 1), dtype=np.int64)
        pairs = np.zeros((max(S, 1), 2), dtype=np.int32)
        npairs = C.c_int32()
        ndone = C.c_int32()
        st = self.lib.pa_append_batch(self.handle, _i32p(tables), maxb, _i32p(nb), S, _i64p(slots),
                                      _i32p(pairs), C.byref(npairs), C.byref(ndone))
        check(self.lib, st, ndone.value)
        return slots[:S], pairs[: npairs.value].copy()

    def fork(self, parent_table: np.ndarray, n_tokens: int, child_table: np.ndarray) -> None:
        assert parent_table.dtype == np.int32 and child_table.dtype == np.int32
        check(self.lib, self.lib.pa_seq_fork(self.handle, _i32p(parent_table), int(n_tokens),
                                             _i32p(child_table), child_table.shape[-1]))

    def free_seq(self, table: np.ndarray, n_tokens: int) -> None:
        assert table.dtype == np.int32
        check(self.lib, self.lib.pa_seq_free(self.handle, _i32p(table), int(n_tokens)))

    def seq_reorder(self, tables: np.ndarray, lens: np.ndarray, parents) -> Tuple[np.ndarray, np.ndarray]:
        """Beam selection: new sequence i continues old sequence parents[i]
        (fork), then every old table is freed.  Returns (new tables int32
        [S_new][maxb], new lengths int32 [S_new])."""
        assert tables.dtype == np.int32 and tables.flags.c_contiguous and tables.ndim == 2
        S_old, maxb = tables.shape
        ln = _as_i32(lens)
        par = _as_i32(parents)
        S_new = int(par.shape[0])
        out = np.empty((max(S_new, 1), maxb), dtype=np.int32)
        out_lens = np.empty(max(S_new, 1), dtype=np.int32)
        check(self.lib, self.lib.pa_seq_reorder(self.handle, _i32p(tables), _i32p(ln), S_old, maxb, _i32p(par), S_new,
                                                _i32p(out), _i32p(out_lens)))
        return out[:S_new], out_lens[:S_new]

    def prefix_groups(self, tables: np.ndarray, lens):
        """Runs of sequences sharing leading blocks (pa_prefix_groups).
        Returns (group_start int32 [n+1], group_len int32 [n], seq_group int32
        [S], max_group, max_shared, max_suffix)."""
        assert tables.dtype == np.int32 and tables.flags.c_contiguous and tables.ndim == 2
        S, maxb = tables.shape
        ln = _as_i32(lens)
        gs = np.zeros(S + 1, dtype=np.int32)
        gl = np.zeros(max(S, 1), dtype=np.int32)
        sg = np.zeros(max(S, 1), dtype=np.int32)
        ng, mg, ms, mx = C.c_int32(), C.c_int32(), C.c_int32(), C.c_int32()
        check(self.lib, self.lib.pa_prefix_groups(self.handle, _i32p(tables), _i32p(ln), S, maxb, _i32p(gs), _i32p(gl),
                                                  _i32p(sg), C.byref(ng), C.byref(mg), C.byref(ms), C.byref(mx)))
        n = ng.value
        return gs[: n + 1].copy(), gl[:n].copy(), sg[:S].copy(), mg.value, ms.value, mx.value

    def validate_step(self, tables: np.ndarray, lens, slots=None) -> None:
        """Debug check of a step's tables, lengths and slots against the
        manager (pa_validate_step); raises PAError naming the first bad
        sequence (attribute ``bad_seq``)."""
        assert tables.dtype == np.int32 and tables.flags.c_contiguous and tables.ndim == 2
        S, maxb = tables.shape
        ln = _as_i32(lens)
        sl = None if slots is None else np.ascontiguousarray(slots, dtype=np.int64)
        bad = C.c_int32(-1)
        st = self.lib.pa_validate_step(self.handle, _i32p(tables), maxb, _i32p(ln), S,
                                       None if sl is None else _i64p(sl), C.byref(bad))
        if st != _abi.PA_OK:
            err = _abi.PAError(st, self.lib.pa_last_error().decode(errors="replace"))
            err.bad_seq = bad.value
            raise err

    def move_blocks(self, to: "Pool", tables: np.ndarray, lens) -> np.ndarray:
        """Swap a group of sequences from this pool to ``to`` (host manager):
        ``tables`` (int32 [S][maxb]) are rewritten in place to name blocks of
        ``to``.  Returns the (old, new) block pairs, int32 [N][2]."""
        assert tables.dtype == np.int32 and tables.flags.c_contiguous and tables.ndim == 2
        S, maxb = tables.shape
        ln = _as_i32(lens)
        cap = int(S * maxb)
        pairs = np.zeros((max(cap, 1), 2), dtype=np.int32)
        n = C.c_int32()
        check(self.lib, self.lib.pa_move_blocks(self.handle, to.handle, _i32p(tables), _i32p(ln), S, maxb,
                                                _i32p(pairs), cap, C.byref(n)))
        return pairs[: n.value].copy()

    # ---- device operations -------------------------------------------------------
    def write_kv(self, layer: int, k, v, slot_mapping, stream=None) -> None:
        """k, v: device [S][Hkv][d] of the pool dtype; slot_mapping: device int64 [S]."""
        S = int(slot_mapping.shape[0])
        check(self.lib, self.lib.pa_write_kv(self.handle, layer, _ptr(k), _ptr(v), _ptr(slot_mapping), S,
                                             _stream_handle(stream)))

    def copy_blocks(self, pairs, stream=None) -> None:
        """pairs: device int32 [N][2]."""
        N = int(pairs.shape[0])
        if N == 0:
            return
        check(self.lib, self.lib.pa_copy_blocks(self.handle, _ptr(pairs), N, _stream_handle(stream)))

    def swap_blocks(self, to: "Pool", pairs, stream=None) -> None:
        """pairs: device int32 [N][2] (block of this pool, block of ``to``)."""
        N = int(pairs.shape[0])
        if N == 0:
            return
        check(self.lib, self.lib.pa_swap_blocks(self.handle, to.handle, _ptr(pairs), N, _stream_handle(stream)))

    def stream_tiles(self, layer: int, block_tables, context_lens, max_ctx: int, checksum, stream=None) -> None:
        """Read the key/value rows decode attention would read (pa_stream_tiles);
        checksum: device int32/uint32 [1], XORed into."""
        S = int(context_lens.shape[0])
        maxb = int(block_tables.shape[1])
        check(self.lib, self.lib.pa_stream_tiles(self.handle, layer, _ptr(block_tables), maxb, _ptr(context_lens), S,
                                                 int(max_ctx), _ptr(checksum), _stream_handle(stream)))

    def workspace_bytes(self, S: int, Hq: int, max_ctx: int) -> int:
        return int(self.lib.pa_decode_workspace_bytes(self.handle, S, Hq, max_ctx))

    def decode_attention(self, layer: int, out, q, block_tables, context_lens, max_ctx: int, scale: float,
                         workspace=None, stream=None) -> None:
        """out, q: device [S][Hq][d]; block_tables: device int32 [S][maxb];
        context_lens: device int32 [S]; workspace: device uint8 tensor from
        ``decode_workspace`` (or None when none is needed)."""
        S, Hq = int(q.shape[0]), int(q.shape[1])
        maxb = int(block_tables.shape[1])
        ws_ptr, ws_bytes = (0, 0) if workspace is None else (_ptr(workspace), int(workspace.numel()))
        check(self.lib, self.lib.pa_decode_attention(
            self.handle, layer, _ptr(out), _ptr(q), S, Hq, _ptr(block_tables), maxb, _ptr(context_lens),
            int(max_ctx), C.c_float(scale), C.c_void_p(ws_ptr or None), C.c_size_t(ws_bytes),
            _stream_handle(stream)))

    def multi_query_attention(self, layer: int, out, q, q_start, block_tables, context_lens, max_ctx: int,
                              max_q: int, scale: float, workspace=None, stream=None,
                              host_context_lens=None) -> None:
        """out, q: device [T][Hq][d]; q_start: device int32 [S+1] (queries of
        sequence s are rows q_start[s] .. q_start[s+1]-1, its last positions);
        block_tables: device int32 [S][maxb]; context_lens: device int32 [S].
        With ``host_context_lens`` (host int32 [S], equal to context_lens)
        the partitions run longest first where the shape allows
        (pa_multi_query_attention_ordered)."""
        T, Hq = int(q.shape[0]), int(q.shape[1])
        S = int(q_start.shape[0]) - 1
        maxb = int(block_tables.shape[1])
        ws_ptr, ws_bytes = (0, 0) if workspace is None else (_ptr(workspace), int(workspace.numel()))
        if host_context_lens is not None:
            hl = np.ascontiguousarray(host_context_lens, dtype=np.int32)
            if hl.shape != (S,):
                raise ValueError("host_context_lens must hold one length per sequence")
            check(self.lib, self.lib.pa_multi_query_attention_ordered(
                self.handle, layer, _ptr(out), _ptr(q), _ptr(q_start), T, S, Hq, _ptr(block_tables), maxb,
                _ptr(context_lens), hl.ctypes.data, int(max_ctx), int(max_q), C.c_float(scale),
                C.c_void_p(ws_ptr or None), C.c_size_t(ws_bytes), _stream_handle(stream)))
            return
        check(self.lib, self.lib.pa_multi_query_attention(
            self.handle, layer, _ptr(out), _ptr(q), _ptr(q_start), T, S, Hq, _ptr(block_tables), maxb,
            _ptr(context_lens), int(max_ctx), int(max_q), C.c_float(scale), C.c_void_p(ws_ptr or None),
            C.c_size_t(ws_bytes), _stream_handle(stream)))

    def grouped_workspace_bytes(self, S: int, Hq: int, max_ctx: int, n_groups: int, max_group: int,
                                max_shared: int, max_suffix: int) -> int:
        return int(self.lib.pa_decode_grouped_workspace_bytes(self.handle, S, Hq, max_ctx, n_groups, max_group,
                                                              max_shared, max_suffix))

    def decode_attention_grouped(self, layer: int, out, q, block_tables, context_lens, max_ctx: int, group_start,
                                 group_len, seq_group, max_group: int, max_shared: int, max_suffix: int,
                                 scale: float, workspace, k=None, v=None, slot_mapping=None, stream=None,
                                 host_group_len=None) -> None:
        """Decode attention reading each group's shared prefix once (see
        pa_decode_attention_grouped); with k, v, slot_mapping the step's
        cache write is done in the same pass.  group_start: device int32
        [n_groups+1]; group_len: device int32 [n_groups]; seq_group: device
        int32 [S].  With ``host_group_len`` (host int32 [n_groups], equal to
        group_len) the group pass runs longest first
        (pa_decode_attention_grouped_ordered)."""
        S, Hq = int(q.shape[0]), int(q.shape[1])
        maxb = int(block_tables.shape[1])
        ng = int(group_start.shape[0]) - 1
        kp = _ptr(k) if k is not None else None
        vp = _ptr(v) if v is not None else None
        sp = _ptr(slot_mapping) if slot_mapping is not None else None
        if host_group_len is not None:
            hg = np.ascontiguousarray(host_group_len, dtype=np.int32)
            if hg.shape != (ng,):
                raise ValueError("host_group_len must hold one length per group")
            check(self.lib, self.lib.pa_decode_attention_grouped_ordered(
                self.handle, layer, C.c_void_p(kp), C.c_void_p(vp), C.c_void_p(sp), _ptr(out), _ptr(q), S, Hq,
                _ptr(block_tables), maxb, _ptr(context_lens), int(max_ctx), _ptr(group_start), _ptr(group_len),
                _ptr(seq_group), hg.ctypes.data, ng, int(max_group), int(max_shared), int(max_suffix),
                C.c_float(scale), _ptr(workspace), C.c_size_t(int(workspace.numel())), _stream_handle(stream)))
            return
        check(self.lib, self.lib.pa_decode_attention_grouped(
            self.handle, layer, C.c_void_p(kp), C.c_void_p(vp), C.c_void_p(sp), _ptr(out), _ptr(q), S, Hq,
            _ptr(block_tables), maxb, _ptr(context_lens), int(max_ctx), _ptr(group_start), _ptr(group_len),
            _ptr(seq_group), ng, int(max_group), int(max_shared), int(max_suffix), C.c_float(scale), _ptr(workspace),
            C.c_size_t(int(workspace.numel())), _stream_handle(stream)))

    def write_kv_decode_attention(self, layer: int, k, v, slot_mapping, out, q, block_tables, context_lens,
                                  max_ctx: int, scale: float, workspace=None, stream=None) -> None:
        """write_kv then decode_attention for one layer in one pass (see
        pa_write_kv_decode_attention)."""
        S, Hq = int(q.shape[0]), int(q.shape[1])
        maxb = int(block_tables.shape[1])
        ws_ptr, ws_bytes = (0, 0) if workspace is None else (_ptr(workspace), int(workspace.numel()))
        check(self.lib, self.lib.pa_write_kv_decode_attention(
            self.handle, layer, _ptr(k), _ptr(v), _ptr(slot_mapping), _ptr(out), _ptr(q), S, Hq,
            _ptr(block_tables), maxb, _ptr(context_lens), int(max_ctx), C.c_float(scale),
            C.c_void_p(ws_ptr or None), C.c_size_t(ws_bytes), _stream_handle(stream)))

    def decode_attention_ordered(self, layer: int, out, q, block_tables, context_lens, host_context_lens,
                                 max_ctx: int, scale: float, workspace=None, k=None, v=None, slot_mapping=None,
                                 stream=None) -> None:
        """decode_attention (or, with k, v and slot_mapping, the fused
        write_kv_decode_attention) with the context partitions launched
        longest first; ``host_context_lens`` is a host int32 array equal to
        ``context_lens`` (see pa_decode_attention_ordered)."""
        S, Hq = int(q.shape[0]), int(q.shape[1])
        maxb = int(block_tables.shape[1])
        hl = np.ascontiguousarray(host_context_lens, dtype=np.int32)
        if hl.shape != (S,):
            raise ValueError("host_context_lens must hold one length per sequence")
        ws_ptr, ws_bytes = (0, 0) if workspace is None else (_ptr(workspace), int(workspace.numel()))
        opt = (lambda t: None if t is None else C.c_void_p(_ptr(t)))
        check(self.lib, self.lib.pa_decode_attention_ordered(
            self.handle, layer, opt(k), opt(v), opt(slot_mapping), _ptr(out), _ptr(q), S, Hq,
            _ptr(block_tables), maxb, _ptr(context_lens), hl.ctypes.data, int(max_ctx), C.c_float(scale),
            C.c_void_p(ws_ptr or None), C.c_size_t(ws_bytes), _stream_handle(stream)))


def decode_attention_ordered_noalloc(pool: Pool, layer: int, out, q, block_tables, context_lens, host_context_lens,
                                     max_ctx: int, scale: float, k=None, v=None, slot_mapping=None,
                                     stream=None) -> None:
    """pa_decode_attention_ordered_noalloc: as Pool.decode_attention_ordered,
    with the partial results in the library's static device scratch."""
    S, Hq = int(q.shape[0]), int(q.shape[1])
    maxb = int(block_tables.shape[1])
    hl = np.ascontiguousarray(host_context_lens, dtype=np.int32)
    if hl.shape != (S,):
        raise ValueError("host_context_lens must hold one length per sequence")
    opt = (lambda t: None if t is None else C.c_void_p(_ptr(t)))
    check(pool.lib, pool.lib.pa_decode_attention_ordered_noalloc(
        pool.handle, layer, opt(k), opt(v), opt(slot_mapping), _ptr(out), _ptr(q), S, Hq, _ptr(block_tables), maxb,
        _ptr(context_lens), hl.ctypes.data, int(max_ctx), C.c_float(scale), _stream_handle(stream)))


def multi_query_workspace(pool: Pool, S: int, Hq: int, max_ctx: int, max_q: int, device="cuda", stream=None):
    """A zero-initialised workspace for ``pool.multi_query_attention``."""
    import torch
    nbytes = int(pool.lib.pa_multi_query_workspace_bytes(pool.handle, S, Hq, max_ctx, max_q))
    if nbytes == 0:
        return None
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    check(pool.lib, pool.lib.pa_decode_workspace_init(_ptr(ws), nbytes, _stream_handle(stream)))
    return ws


def decode_workspace(pool: Pool, S: int, Hq: int, max_ctx: int, device="cuda", stream=None):
    """A zero-initialised workspace for ``pool.decode_attention`` at these
    sizes (None if the launch needs none)."""
    import torch
    nbytes = pool.workspace_bytes(S, Hq, max_ctx)
    if nbytes == 0:
        return None
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    check(pool.lib, pool.lib.pa_decode_workspace_init(_ptr(ws), nbytes, _stream_handle(stream)))
    return ws
