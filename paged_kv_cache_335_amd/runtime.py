"""One paged KV cache on one GPU, driven step by step.

Glue only: the host block manager (C) decides blocks, slots and copies; one
packed host-to-device copy per step carries the step's metadata; the HIP
library applies copies, writes, table growth and decode.  Torch provides the
device buffers, pinned staging memory and the stream.

A decode step for a batch of live sequences:
  1. pa_bm_append_batch: one new slot per sequence (new block when the tail
     is full, copy-on-write pair when the tail is shared and partly filled);
  2. one async copy of [slots | row ids | positions | lengths] to the device;
  3. pa_block_copy for copy-on-write pairs (if any);
  4. pa_kv_append: device table rows follow the growth and the new tokens'
     K/V go into their slots, in one launch;
  5. pa_decode: attention over the grown contexts.

With share_prefixes=True the step also exports the batch's prefix groups
(runs of table rows whose leading full blocks are the same physical
blocks, e.g. the samples forked from one prompt) in the same staging copy,
and decode reads each group's shared blocks once for all of its members
(pa_decode_shared).

Every device operation of a call, allocations and copies included, runs
on the stream the call names (the current stream by default), so a caller
may drive the cache from a side stream.

Preemption by swapping: swap_out(seq) moves a sequence's blocks to a pinned
host pool and frees them on the device; swap_in(seq) brings them back into
new device blocks and rewrites the sequence's table row.  While any
sequence is swapped out, decode takes the list of resident sequences.
"""
import ctypes

import numpy as np
import torch

from . import (PA_OK, PA_SWAP_IN, PA_SWAP_OUT, PagedKVError, alloc_host_pools, alloc_pools,
               pa_block_copy, pa_block_swap, pa_decode, pa_decode_partition_tokens,
               pa_decode_shared, pa_decode_shared_workspace_bytes, pa_decode_step,
               pa_decode_workspace_bytes, pa_extend, pa_kv_append)
from .block_manager import BlockManager

# Staging for the per-step metadata: a ring of pinned host buffers, each
# copied to its own device buffer.  An event is recorded only after the last
# copy of each group of _GROUP buffers (any event between two kernels delays
# the second by a few microseconds), and the host waits on a group's event
# only when it comes back to that group a lap later.
_RING = 32
_GROUP = 8

# --- fence-free stream events ---------------------------------------------------
# A default HIP event performs a system-scope release when it is recorded:
# caches are written back and invalidated, and on this GPU the kernel after
# each record started about 5 us late.  Events that only order work on the
# device, time it, or tell the host that a host-to-device copy has finished
# reading its source need no such fence.
_HIP_EVENT_DISABLE_TIMING = 0x2
_HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000
_hip = None


def _hip_runtime():
    """The HIP runtime torch already loaded (opened by soname, so no second
    copy is mapped into the process)."""
    global _hip
    if _hip is None:
        lib = ctypes.CDLL("libamdhip64.so.7")
        vp = ctypes.c_void_p
        lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
        lib.hipEventRecord.argtypes = [vp, vp]
        lib.hipEventSynchronize.argtypes = [vp]
        lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
        lib.hipEventDestroy.argtypes = [vp]
        _hip = lib
    return _hip


class DeviceEvent:
    """A HIP event recorded without a system-scope fence."""

    def __init__(self, timing=False):
        hip = _hip_runtime()
        flags = _HIP_EVENT_DISABLE_SYSTEM_FENCE | (0 if timing else _HIP_EVENT_DISABLE_TIMING)
        self._ev = ctypes.c_void_p()
        st = hip.hipEventCreateWithFlags(ctypes.byref(self._ev), flags)
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({st})")

    def record(self, stream):
        st = _hip_runtime().hipEventRecord(self._ev, ctypes.c_void_p(stream.cuda_stream))
        if st != 0:
            raise RuntimeError(f"hipEventRecord failed ({st})")

    def synchronize(self):
        st = _hip_runtime().hipEventSynchronize(self._ev)
        if st != 0:
            raise RuntimeError(f"hipEventSynchronize failed ({st})")

    def elapsed_ms(self, end):
        ms = ctypes.c_float()
        st = _hip_runtime().hipEventElapsedTime(ctypes.byref(ms), self._ev, end._ev)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st})")
        return float(ms.value)

    def __del__(self):
        if getattr(self, "_ev", None) and _hip is not None:
            _hip.hipEventDestroy(self._ev)
            self._ev = None


class PagedKVCache:
    def __init__(self, num_blocks, num_kv_heads, head_dim, max_seqs, table_width,
                 block_size=16, dtype=torch.bfloat16, shuffle_seed=0, device="cuda",
                 host_blocks=0, share_prefixes=False, max_group=4):
        self.B = block_size
        self.max_group = max_group  # members per prefix group (16 // query heads per kv head)
        self.num_kv_heads = num_kv_heads
        self.head_dim = head_dim
        self.max_seqs = max_seqs
        self.width = table_width
        self.dtype = dtype
        self.device = torch.device(device)
        self.bm = BlockManager(num_blocks, block_size, shuffle_seed)
        # dtype torch.uint8: 8-bit pools (E4M3 codes + per-token scales)
        self.k_pool, self.v_pool = alloc_pools(num_blocks, num_kv_heads, head_dim, block_size,
                                               dtype, self.device)
        self.tables = torch.zeros((max_seqs, table_width), dtype=torch.int32, device=self.device)
        # device lengths of the latest step (a view into its staging buffer)
        self.lens = torch.zeros(max_seqs, dtype=torch.int32, device=self.device)
        self.host_lens = np.zeros(max_seqs, dtype=np.int32)
        self.host_k = self.host_v = None
        if host_blocks:
            self.host_k, self.host_v = alloc_host_pools(host_blocks, self.k_pool, self.v_pool)
            st = self.bm.set_host_blocks(host_blocks)
            if st != PA_OK:
                raise PagedKVError(st, "pa_bm_set_host_blocks")
        self.rows = {}          # sequence id -> row of the device table
        self.row_seqs = []      # sequence id of each table row
        self.swapped = set()    # sequences whose blocks are in the host pool
        self.share_prefixes = share_prefixes
        self.groups = None      # device (group_start, shared_blocks) of the latest step
        self.num_groups = 0
        self._ring = None
        self._ring_events = [None] * (_RING // _GROUP)
        self._ring_pos = 0
        self._ws = None
        self._ws_key = None     # sizes the workspace was last sized for
        self._ws_view = None
        self._rows_cache = None  # (row sequence ids, ones) as int32 arrays
        # decode steps: device lengths alternate between two buffers (a step
        # reads one and writes the other)
        self._lens_bufs = [torch.zeros(max_seqs, dtype=torch.int32, device=self.device)
                           for _ in range(2)]
        self._step_groups = None   # (host gs, host sb, device gs, device sb)

    # --- sequences ------------------------------------------------------
    def _stream(self, stream):
        return stream or torch.cuda.current_stream(self.device)

    def add_sequence(self) -> int:
        if len(self.rows) >= self.max_seqs:
            raise ValueError("table rows exhausted")
        s = self.bm.add_seq()
        self.rows[s] = len(self.rows)
        self.row_seqs.append(s)
        return s

    def fork(self, parent: int, stream=None) -> int:
        """A new sequence sharing every block of ``parent``: its device table
        row is copied from the parent's on ``stream``, after any earlier
        growth of that row enqueued there."""
        st, child = self.bm.fork(parent)
        if st != PA_OK:
            raise PagedKVError(st, "pa_bm_fork")
        if len(self.rows) >= self.max_seqs:
            raise ValueError("table rows exhausted")
        r = len(self.rows)
        self.rows[child] = r
        self.row_seqs.append(child)
        self.host_lens[r] = self.host_lens[self.rows[parent]]
        stream = self._stream(stream)
        with torch.cuda.stream(stream):
            self.tables[r].copy_(self.tables[self.rows[parent]])
            self.lens = torch.from_numpy(self.host_lens.copy()).to(self.device, non_blocking=False)
        return child

    # --- staging ----------------------------------------------------------
    def _staging(self, nbytes, stream):
        if self._ring is None or self._ring[0][0].numel() < nbytes:
            if self._ring is not None:
                # the old buffers may still be read by copies and kernels on
                # any stream a previous call named
                torch.cuda.synchronize(self.device)
            with torch.cuda.stream(stream):
                self._ring = [(torch.empty(nbytes, dtype=torch.uint8, pin_memory=True),
                               torch.empty(nbytes, dtype=torch.uint8, device=self.device))
                              for _ in range(_RING)]
            self._ring_events = [None] * (_RING // _GROUP)
            self._ring_pos = 0
        i = self._ring_pos
        self._ring_pos = (i + 1) % _RING
        if i % _GROUP == 0:
            ev = self._ring_events[i // _GROUP]
            if ev is not None:
                ev.synchronize()  # every copy of this group's previous lap has run
        return i

    def append(self, seqs, n_tokens, k_new, v_new, stream=None):
        """Append n_tokens[i] tokens to seqs[i]; k_new/v_new [sum n][Hkv][d].
        Returns the number of copy-on-write pairs applied."""
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        n_tokens = np.ascontiguousarray(n_tokens, dtype=np.int32)
        st, slots, sq, pos, pairs = self.bm.append_batch(seqs, n_tokens)
        if st != PA_OK:
            raise PagedKVError(st, "pa_bm_append_batch")
        T = len(slots)
        rows = np.fromiter((self.rows[int(s)] for s in seqs), dtype=np.int32, count=len(seqs))
        row_of_tok = np.repeat(rows, n_tokens)
        self.host_lens[rows] += n_tokens
        S = len(self.rows)
        gs = sb = None
        if self.share_prefixes and not self.swapped:
            st, gs, sb = self.bm.prefix_groups(self.row_seqs, self.max_group)
            if st != PA_OK:
                raise PagedKVError(st, "pa_bm_prefix_groups")
        G = 0 if gs is None else len(sb)
        o_sq = T * 8
        o_pos = o_sq + T * 4
        o_len = o_pos + T * 4
        o_gs = o_len + S * 4
        o_sb = o_gs + (G + 1) * 4
        end = o_sb + G * 4
        stream = self._stream(stream)
        i = self._staging(max(end, 64), stream)
        host, dev = self._ring[i]
        hv = host.numpy()
        hv[:o_sq].view(np.int64)[:] = slots
        hv[o_sq:o_pos].view(np.int32)[:] = row_of_tok
        hv[o_pos:o_len].view(np.int32)[:] = pos
        hv[o_len:o_gs].view(np.int32)[:] = self.host_lens[:S]
        if G:
            hv[o_gs:o_sb].view(np.int32)[:] = gs
            hv[o_sb:end].view(np.int32)[:] = sb
        with torch.cuda.stream(stream):
            dev[:end].copy_(host[:end], non_blocking=True)
            if i % _GROUP == _GROUP - 1:
                # after the group's last copy: the host may refill the group once it fires
                g = i // _GROUP
                ev = self._ring_events[g] or DeviceEvent()
                ev.record(stream)
                self._ring_events[g] = ev
            d_slots = dev[:o_sq].view(torch.int64)
            d_rows = dev[o_sq:o_pos].view(torch.int32)
            d_pos = dev[o_pos:o_len].view(torch.int32)
            self.lens = dev[o_len:o_gs].view(torch.int32)
            if G:
                self.groups = (dev[o_gs:o_sb].view(torch.int32), dev[o_sb:end].view(torch.int32))
                self.num_groups = G
            if len(pairs):
                d_pairs = torch.from_numpy(np.ascontiguousarray(pairs)).to(self.device,
                                                                           non_blocking=False)
                pa_block_copy(self.k_pool, self.v_pool, d_pairs, stream=stream)
            pa_kv_append(self.k_pool, self.v_pool, k_new, v_new, d_slots, self.tables, d_rows,
                         d_pos, stream=stream)
        return len(pairs)

    # --- one decode step in one launch ------------------------------------------
    def step(self, q, k_new, v_new, out=None, scale=None, partition_tokens=0, stream=None):
        """One decode step of every live sequence (rows in table order): the
        block manager gives each sequence one new slot, then one launch
        (pa_decode_step) stores the new tokens k_new/v_new [S][Hkv][d], grows
        the tables and lengths, and decodes q [S][Hq][d] over the grown
        contexts.  The host sends only each token's block id, with the
        launch's arguments; copy-on-write copies (after a fork) run first.
        bf16 and 8-bit pools; fp32 pools take append + decode."""
        if self.swapped:
            raise ValueError("sequences are swapped out")
        stream = self._stream(stream)
        S = len(self.rows)
        if self.k_pool.dtype == torch.float32:
            self.append(np.asarray(self.row_seqs, np.int32), np.ones(S, np.int32), k_new, v_new,
                        stream=stream)
            return self.decode(q, out=out, scale=scale, partition_tokens=partition_tokens,
                               stream=stream)
        seqs, ones = self._row_arrays()
        st, slots, _, pos, pairs = self.bm.append_batch(seqs, ones)
        if st != PA_OK:
            raise PagedKVError(st, "pa_bm_append_batch")
        # every token's block is given (the kernel writes its table entry)
        nb = (slots // self.B).astype(np.int32)
        lens_in = self.lens[:S]
        lens_out = self._lens_bufs[0]
        if lens_out.data_ptr() == lens_in.data_ptr():
            lens_out = self._lens_bufs[1]
        self.host_lens[:S] += 1
        gs = sb = None
        if self.share_prefixes:
            st, hgs, hsb = self.bm.prefix_groups(seqs, self.max_group)
            if st != PA_OK:
                raise PagedKVError(st, "pa_bm_prefix_groups")
            cached = self._step_groups
            if cached is None or not (np.array_equal(cached[0], hgs) and
                                      np.array_equal(cached[1], hsb)):
                with torch.cuda.stream(stream):
                    cached = (hgs, hsb, torch.from_numpy(hgs).to(self.device, non_blocking=False),
                              torch.from_numpy(hsb).to(self.device, non_blocking=False))
                self._step_groups = cached
            gs, sb = cached[2], cached[3]
        scale = self.head_dim ** -0.5 if scale is None else scale
        if len(pairs):
            with torch.cuda.stream(stream):
                d_pairs = torch.from_numpy(np.ascontiguousarray(pairs)).to(self.device,
                                                                           non_blocking=False)
            pa_block_copy(self.k_pool, self.v_pool, d_pairs, stream=stream)
        # the launch takes the stream explicitly and the output is allocated
        # on it, so no stream context is needed around the launch (one costs
        # ~10 us of host time a step)
        if out is None:
            with torch.cuda.stream(stream):
                out = torch.empty_like(q)
        ws = self.workspace(q.shape[1], partition_tokens, stream)
        out = pa_decode_step(q, self.k_pool, self.v_pool, k_new, v_new, self.tables[:S],
                             lens_in, lens_out[:S], nb, scale, out=out,
                             group_start=gs, shared_blocks=sb,
                             partition_tokens=partition_tokens, workspace=ws, stream=stream)
        self.lens = lens_out
        self.groups = None if gs is None else (gs, sb)
        return out

    # --- preemption by swapping ------------------------------------------------
    def _swap(self, seq, out, stream):
        st, pairs = (self.bm.swap_out if out else self.bm.swap_in)(seq)
        if st != PA_OK:
            raise PagedKVError(st, "pa_bm_swap_out" if out else "pa_bm_swap_in")
        stream = stream or torch.cuda.current_stream(self.device)
        if len(pairs):
            d_pairs = torch.from_numpy(np.ascontiguousarray(pairs)).to(self.device)
            with torch.cuda.stream(stream):
                pa_block_swap(self.k_pool, self.v_pool, self.host_k, self.host_v, d_pairs,
                              PA_SWAP_OUT if out else PA_SWAP_IN, stream=stream)
        return pairs

    def swap_out(self, seq, stream=None):
        """Copy seq's blocks to the host pool and free them on the device.
        Returns the (device block, host block) pairs."""
        pairs = self._swap(seq, True, stream)
        self.swapped.add(seq)
        return pairs

    def swap_in(self, seq, stream=None):
        """Bring seq's blocks back into new device blocks and rewrite its
        table row.  Returns the (host block, device block) pairs."""
        pairs = self._swap(seq, False, stream)
        self.swapped.discard(seq)
        st, table, n = self.bm.block_table(seq)
        row = self.rows[seq]
        with torch.cuda.stream(self._stream(stream)):
            self.tables[row, :len(table)].copy_(torch.tensor(table, dtype=torch.int32),
                                                non_blocking=False)
        return pairs

    # --- decode -------------------------------------------------------------
    def workspace(self, num_q_heads, partition_tokens=0, stream=None):
        S = len(self.rows)
        key = (S, num_q_heads, partition_tokens, self.share_prefixes)
        if self._ws_key == key:
            return self._ws_view
        query = pa_decode_shared_workspace_bytes if self.share_prefixes else \
            pa_decode_workspace_bytes
        need = query(self.k_pool, self.v_pool, S, num_q_heads, self.width, partition_tokens)
        if need and (self._ws is None or self._ws.numel() < need):
            if self._ws is not None:
                torch.cuda.synchronize(self.device)  # the old workspace may still be in use
            with torch.cuda.stream(self._stream(stream)):
                self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        self._ws_key, self._ws_view = key, (self._ws if need else None)
        return self._ws_view

    def _row_arrays(self):
        """The table rows' sequence ids and a ones vector, as int32 arrays
        (rebuilt only when rows change)."""
        if self._rows_cache is None or len(self._rows_cache[0]) != len(self.row_seqs):
            self._rows_cache = (np.asarray(self.row_seqs, np.int32),
                                np.ones(len(self.row_seqs), np.int32))
        return self._rows_cache

    def partition_tokens(self, num_q_heads, partition_tokens=0):
        return pa_decode_partition_tokens(self.k_pool, self.v_pool, len(self.rows), num_q_heads,
                                          self.width, partition_tokens)

    def decode_seqs(self, q, seqs, out=None, scale=None, partition_tokens=0, stream=None):
        """Attention of q [len(seqs)][Hq][d] over the contexts of the given
        resident sequences (tables exported by the block manager and copied
        to the device for this call)."""
        tables, lens = self.bm.export(np.asarray(seqs, np.int32), self.width, pad_block=0)
        scale = self.head_dim ** -0.5 if scale is None else scale
        stream = self._stream(stream)
        # uploads and the workspace belong to `stream`, so their memory is
        # not reused before the kernels that read it there have run
        with torch.cuda.stream(stream):
            d_tables = torch.from_numpy(tables).to(self.device, non_blocking=False)
            d_lens = torch.from_numpy(lens).to(self.device, non_blocking=False)
            return pa_decode(q, self.k_pool, self.v_pool, d_tables, d_lens, scale, out=out,
                             partition_tokens=partition_tokens, stream=stream)

    def extend(self, seqs, n_tokens, q, k_new, v_new, out=None, scale=None, stream=None):
        """Chunked prefill / extend: append n_tokens[i] tokens to seqs[i]
        (slot write), then causal attention of their queries q [sum n][Hq][d]
        over each sequence's context.  Returns out like q."""
        stream = stream or torch.cuda.current_stream(self.device)
        self.append(seqs, n_tokens, k_new, v_new, stream=stream)
        tables, lens = self.bm.export(np.asarray(seqs, np.int32), self.width, pad_block=0)
        q_start = np.concatenate([[0], np.cumsum(n_tokens)]).astype(np.int32)
        scale = self.head_dim ** -0.5 if scale is None else scale
        with torch.cuda.stream(stream):
            d_tables = torch.from_numpy(tables).to(self.device)
            d_lens = torch.from_numpy(lens).to(self.device)
            d_qs = torch.from_numpy(q_start).to(self.device)
            return pa_extend(q, self.k_pool, self.v_pool, d_qs, d_tables, d_lens, scale,
                             out=out, stream=stream)

    def decode(self, q, out=None, scale=None, partition_tokens=0, stream=None):
        """Attention of q [S][Hq][d] (rows in table order) over every live
        sequence's context (none may be swapped out: use decode_seqs)."""
        if self.swapped:
            raise ValueError("sequences are swapped out; decode the resident ones with "
                             "decode_seqs")
        S = len(self.rows)
        scale = self.head_dim ** -0.5 if scale is None else scale
        stream = self._stream(stream)
        with torch.cuda.stream(stream):
            ws = self.workspace(q.shape[1], partition_tokens)
            if self.share_prefixes and self.groups is not None:
                return pa_decode_shared(q, self.k_pool, self.v_pool, self.tables[:S],
                                        self.lens[:S], scale, self.groups[0], self.groups[1],
                                        out=out, partition_tokens=partition_tokens, workspace=ws,
                                        stream=stream)
            return pa_decode(q, self.k_pool, self.v_pool, self.tables[:S], self.lens[:S], scale,
                             out=out, partition_tokens=partition_tokens, workspace=ws,
                             stream=stream)
