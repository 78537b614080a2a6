"""ctypes wrapper of the C host block manager (pa_bm_* in include/pa_bm.h).

Marshalling only: free pool, refcounts, tables and copy-on-write decisions
all live in the C library.  Host memory only; usable without a GPU."""
import ctypes

import numpy as np

from . import BMStats, PA_OK, PagedKVError, lib

_vp = ctypes.c_void_p


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_vp)


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, shuffle_seed: int = 0):
        self._lib = lib()
        self._h = self._lib.pa_bm_create(int(num_blocks), int(block_size),
                                         ctypes.c_uint64(int(shuffle_seed)))
        if not self._h:
            raise ValueError("pa_bm_create failed (bad sizes or host memory)")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def close(self):
        if getattr(self, "_h", None):
            self._lib.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    # Each method returns the C status plus its outputs, mirroring the C API;
    # the *_or_raise helpers raise PagedKVError instead.
    def add_seq(self) -> int:
        out = ctypes.c_int32()
        st = self._lib.pa_bm_add_seq(self._h, ctypes.byref(out))
        if st != PA_OK:
            raise PagedKVError(st, "pa_bm_add_seq")
        return out.value

    def fork(self, parent: int):
        out = ctypes.c_int32(-1)
        st = self._lib.pa_bm_fork(self._h, int(parent), ctypes.byref(out))
        return st, out.value

    def append(self, seq: int, n: int):
        """Returns (status, slots list, cow pairs list)."""
        n = int(n)
        slots = np.empty(max(n, 1), np.int64)
        pairs = np.empty(2, np.int32)
        ncow = ctypes.c_int32(0)
        st = self._lib.pa_bm_append(self._h, int(seq), n, _ptr(slots), _ptr(pairs),
                                    ctypes.byref(ncow))
        if st != PA_OK:
            return st, [], []
        return st, slots[:n].tolist(), [tuple(pairs.tolist())] if ncow.value else []

    def append_batch(self, seqs, n_tokens):
        """Returns (status, slots int64[], seq ids int32[], positions int32[],
        cow pairs int32[k][2])."""
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        n_tokens = np.ascontiguousarray(n_tokens, dtype=np.int32)
        total = int(n_tokens.sum()) if len(n_tokens) else 0
        slots = np.empty(max(total, 1), np.int64)
        sq = np.empty(max(total, 1), np.int32)
        pos = np.empty(max(total, 1), np.int32)
        pairs = np.empty((max(len(seqs), 1), 2), np.int32)
        ncow = ctypes.c_int32(0)
        st = self._lib.pa_bm_append_batch(self._h, _ptr(seqs), _ptr(n_tokens), len(seqs),
                                          _ptr(slots), _ptr(sq), _ptr(pos), _ptr(pairs),
                                          ctypes.byref(ncow))
        if st != PA_OK:
            return st, None, None, None, None
        return st, slots[:total], sq[:total], pos[:total], pairs[:ncow.value]

    def free_seq(self, seq: int) -> int:
        return self._lib.pa_bm_free_seq(self._h, int(seq))

    def block_table(self, seq: int):
        """Returns (status, table list, n_tokens)."""
        nb = ctypes.c_int32(0)
        nt = ctypes.c_int32(0)
        st = self._lib.pa_bm_block_table(self._h, int(seq), None, 0, ctypes.byref(nb),
                                          ctypes.byref(nt))
        if st != PA_OK:
            return st, [], 0
        out = np.empty(max(nb.value, 1), np.int32)
        self._lib.pa_bm_block_table(self._h, int(seq), _ptr(out), nb.value, None, None)
        return st, out[:nb.value].tolist(), nt.value

    def export(self, seqs, width: int, pad_block: int = 0):
        """Dense (tables int32 [n][width], lens int32 [n]) for a decode batch."""
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        tables = np.empty((len(seqs), width), np.int32)
        lens = np.empty(len(seqs), np.int32)
        st = self._lib.pa_bm_export(self._h, _ptr(seqs), len(seqs), _ptr(tables), int(width),
                                    int(pad_block), _ptr(lens))
        if st != PA_OK:
            raise PagedKVError(st, "pa_bm_export")
        return tables, lens

    def set_host_blocks(self, n: int) -> int:
        return self._lib.pa_bm_set_host_blocks(self._h, int(n))

    def _swap(self, fn, seq: int):
        nb = ctypes.c_int32(0)
        self._lib.pa_bm_block_table(self._h, int(seq), None, 0, ctypes.byref(nb), None)
        pairs = np.empty((max(nb.value, 1), 2), np.int32)
        n = ctypes.c_int32(0)
        st = fn(self._h, int(seq), _ptr(pairs), ctypes.byref(n))
        if st != PA_OK:
            return st, np.empty((0, 2), np.int32)
        return st, pairs[:n.value]

    def swap_out(self, seq: int):
        """Returns (status, pairs int32 [n][2] = (device block, host block))."""
        return self._swap(self._lib.pa_bm_swap_out, seq)

    def swap_in(self, seq: int):
        """Returns (status, pairs int32 [n][2] = (host block, device block))."""
        return self._swap(self._lib.pa_bm_swap_in, seq)

    def is_swapped(self, seq: int) -> int:
        return int(self._lib.pa_bm_is_swapped(self._h, int(seq)))

    def host_free_list(self):
        n = self._lib.pa_bm_host_free_list(self._h, None, 0)
        out = np.empty(max(n, 1), np.int32)
        self._lib.pa_bm_host_free_list(self._h, _ptr(out), n)
        return out[:n].tolist()

    def prefix_groups(self, seqs, max_members: int):
        """(status, group_start [n_groups + 1], shared_blocks [n_groups]) for a
        decode batch in the order given (pa_bm_prefix_groups)."""
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        n = len(seqs)
        gs = np.zeros(n + 1, np.int32)
        sb = np.zeros(max(n, 1), np.int32)
        k = ctypes.c_int32()
        st = self._lib.pa_bm_prefix_groups(self._h, _ptr(seqs), n, int(max_members), _ptr(gs),
                                           _ptr(sb), ctypes.byref(k))
        return st, gs[:k.value + 1].copy(), sb[:k.value].copy()

    def refcount(self, block: int) -> int:
        return int(self._lib.pa_bm_refcount(self._h, int(block)))

    def refcounts(self):
        return [self.refcount(b) for b in range(self.num_blocks)]

    def free_list(self):
        n = self._lib.pa_bm_free_list(self._h, None, 0)
        out = np.empty(max(n, 1), np.int32)
        self._lib.pa_bm_free_list(self._h, _ptr(out), n)
        return out[:n].tolist()

    def stats(self) -> dict:
        s = BMStats()
        st = self._lib.pa_bm_stats(self._h, ctypes.byref(s))
        if st != PA_OK:
            raise PagedKVError(st, "pa_bm_stats")
        return {name: int(getattr(s, name)) for name, _ in BMStats._fields_}
