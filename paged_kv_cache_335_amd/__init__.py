"""Python binding of libpagedkv (paged KV-cache kernels for MI355X / gfx950).

Argument marshalling only: every step of the path runs in the HIP library.
The functions carry the C names (``pa_decode``, ``pa_kv_write``, ...) and take
torch tensors, passing their device pointers and the current HIP stream.
The library must have been built (``python paged_kv_cache_335_amd/build.py``);
importing this package fails loudly when it is missing.  PyTorch is used for
device memory and streams only.

Layouts (see include/pa.h):
    k_pool  [num_blocks][num_kv_heads][block_size][head_dim]
    v_pool  [num_blocks][num_kv_heads][head_dim][block_size]
    q, out  [num_seqs][num_q_heads][head_dim]
8-bit pools (PA_FP8_E4M3) are uint8: k_pool [num_blocks][num_kv_heads][R_k],
R_k = block_size*(head_dim + 4), holding per (block, kv head) the E4M3 K
codes token-major and then bf16 scales (per 4 slots: 4 K, then 4 V);
v_pool [num_blocks][num_kv_heads][R_v], R_v = block_size*head_dim, holding
the V codes dim-major.  Their q, out, k_new and v_new are bfloat16.
"""
import ctypes
import os

import numpy as np
import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpagedkv.so")

PA_OK, PA_EINVAL, PA_ENOMEM, PA_EHIP, PA_EUNSUPPORTED, PA_ESCRATCH = range(6)
PA_F32, PA_BF16, PA_FP8_E4M3 = 0, 1, 2
PA_SWAP_OUT, PA_SWAP_IN = 0, 1


class PagedKVError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} (status {status})")


class PoolDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class BMStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "num_blocks", "block_size", "free_blocks", "used_blocks", "shared_blocks",
        "live_seqs", "logical_tokens", "logical_blocks", "stored_tokens",
        "allocated_slots", "cow_copies", "enomem_events", "swapped_seqs", "host_blocks",
        "host_free_blocks", "swapped_out_blocks", "swapped_in_blocks")]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python paged_kv_cache_335_amd/build.py` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, vp, sz, f32 = (ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t,
                             ctypes.c_float)
    P = ctypes.POINTER(PoolDesc)
    sigs = {
        "pa_kv_write": (i32, [P, vp, vp, vp, vp, vp, i32, vp]),
        "pa_decode_workspace_bytes": (sz, [P, i32, i32, i32, i32]),
        "pa_decode_partition_tokens": (i32, [P, i32, i32, i32, i32]),
        "pa_decode_piece_tokens": (i32, [P, i32, i32, i32, i32, i64]),
        "pa_decode": (i32, [P, vp, vp, vp, i32, i32, vp, i32, vp, f32, vp, i32, vp, sz, vp]),
        "pa_decode_shared": (i32, [P, vp, vp, vp, i32, i32, vp, i32, vp, f32, vp, i32, i32, vp,
                                   vp, vp, sz, vp]),
        "pa_decode_noalloc": (i32, [P, vp, vp, vp, i32, i32, vp, i32, vp, f32, vp, i32, vp]),
        "pa_decode_step": (i32, [P, vp, vp, vp, vp, vp, i32, i32, vp, i32, vp, vp, vp, f32, vp,
                                 i32, i32, vp, vp, vp, sz, vp]),
        "pa_decode_noalloc_max_bytes": (sz, []),
        "pa_decode_shared_workspace_bytes": (sz, [P, i32, i32, i32, i32]),
        "pa_block_copy": (i32, [P, vp, vp, vp, i32, vp]),
        "pa_table_update": (i32, [vp, i32, i32, vp, vp, vp, i32, vp]),
        "pa_kv_append": (i32, [P, vp, vp, vp, vp, vp, i32, vp, i32, vp, vp, vp]),
        "pa_block_swap": (i32, [P, vp, vp, vp, vp, i32, vp, i32, i32, vp]),
        "pa_extend": (i32, [P, vp, vp, vp, i32, vp, i32, i32, vp, i32, vp, f32, vp, vp, sz, vp]),
        "pa_extend_workspace_bytes": (sz, [P, i32, i32, i32, i32]),
        "pa_probe_sink_bytes": (sz, [i32]),
        "pa_probe_read": (i32, [vp, vp, i32, ctypes.c_uint32, i32, i32, vp, vp]),
        "pa_status_str": (ctypes.c_char_p, [i32]),
        "pa_version": (ctypes.c_char_p, []),
        "pa_bm_create": (vp, [i32, i32, ctypes.c_uint64]),
        "pa_bm_destroy": (None, [vp]),
        "pa_bm_add_seq": (i32, [vp, vp]),
        "pa_bm_fork": (i32, [vp, i32, vp]),
        "pa_bm_append": (i32, [vp, i32, i32, vp, vp, vp]),
        "pa_bm_append_batch": (i32, [vp, vp, vp, i32, vp, vp, vp, vp, vp]),
        "pa_bm_free_seq": (i32, [vp, i32]),
        "pa_bm_block_table": (i32, [vp, i32, vp, i32, vp, vp]),
        "pa_bm_export": (i32, [vp, vp, i32, vp, i32, i32, vp]),
        "pa_bm_refcount": (i32, [vp, i32]),
        "pa_bm_free_list": (i32, [vp, vp, i32]),
        "pa_bm_prefix_groups": (i32, [vp, vp, i32, i32, vp, vp, vp]),
        "pa_bm_stats": (i32, [vp, ctypes.POINTER(BMStats)]),
        "pa_bm_set_host_blocks": (i32, [vp, i32]),
        "pa_bm_swap_out": (i32, [vp, i32, vp, vp]),
        "pa_bm_swap_in": (i32, [vp, i32, vp, vp]),
        "pa_bm_is_swapped": (i32, [vp, i32]),
        "pa_bm_host_free_list": (i32, [vp, vp, i32]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()
EXPORTED = (
    "pa_kv_write", "pa_decode_workspace_bytes", "pa_decode_partition_tokens",
    "pa_decode_piece_tokens", "pa_decode",
    "pa_decode_shared", "pa_decode_shared_workspace_bytes", "pa_decode_step",
    "pa_decode_noalloc",
    "pa_decode_noalloc_max_bytes",
    "pa_block_copy", "pa_table_update", "pa_kv_append", "pa_block_swap", "pa_extend",
    "pa_extend_workspace_bytes",
    "pa_status_str", "pa_probe_sink_bytes", "pa_probe_read",
    "pa_version", "pa_bm_create",
    "pa_bm_destroy", "pa_bm_add_seq", "pa_bm_fork", "pa_bm_append", "pa_bm_append_batch",
    "pa_bm_free_seq", "pa_bm_block_table", "pa_bm_export", "pa_bm_refcount",
    "pa_bm_free_list", "pa_bm_prefix_groups", "pa_bm_stats", "pa_bm_set_host_blocks", "pa_bm_swap_out",
    "pa_bm_swap_in", "pa_bm_is_swapped", "pa_bm_host_free_list")


def lib():
    return _lib


def status_str(status):
    return _lib.pa_status_str(int(status)).decode()


def version():
    return _lib.pa_version().decode()


def _check(status, what):
    if status != PA_OK:
        raise PagedKVError(status, what)


def _dtype_code(t: torch.Tensor):
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.uint8:
        return PA_FP8_E4M3
    raise TypeError(f"pool dtype must be bfloat16, float32 or uint8 (8-bit regions), "
                    f"got {t.dtype}")


def io_dtype(k_pool: torch.Tensor):
    """Element type of q, out, k_new and v_new for a pool."""
    return torch.bfloat16 if k_pool.dtype == torch.uint8 else k_pool.dtype


def fp8_region_bytes(block_size: int, head_dim: int):
    """(K, V) bytes of one (block, kv head) region of an 8-bit pool."""
    return block_size * head_dim + 4 * block_size, block_size * head_dim


def side_by_side(buf: torch.Tensor, rk: int):
    """(k_pool, v_pool) views of one uint8 buffer [num_blocks][num_kv_heads]
    [R_k + R_v] whose (block, kv head) regions hold K (codes and scales) and
    then V: the 8-bit layout the library reads with one contiguous run per
    (block, kv head)."""
    return buf[:, :, :rk], buf[:, :, rk:]


def fp8_pools_side_by_side(k_pool, v_pool, device="cuda"):
    """Copy two-buffer 8-bit pools (arrays or tensors [nb][H][R_k], [nb][H]
    [R_v]) into one side-by-side buffer on `device`; returns its views."""
    k = torch.as_tensor(k_pool)
    v = torch.as_tensor(v_pool)
    buf = torch.empty((k.shape[0], k.shape[1], k.shape[2] + v.shape[2]), dtype=torch.uint8,
                      device=device)
    kv, vv = side_by_side(buf, k.shape[2])
    kv.copy_(k)
    vv.copy_(v)
    return kv, vv


def alloc_pools(num_blocks, num_kv_heads, head_dim, block_size=16, dtype=torch.bfloat16,
                device="cuda"):
    """Uninitialised (k_pool, v_pool) in the library's layout; dtype
    torch.uint8 gives 8-bit (E4M3 + scale) pools, as views of one buffer
    with each (block, kv head)'s K and V regions side by side."""
    if dtype == torch.uint8:
        rk, rv = fp8_region_bytes(block_size, head_dim)
        buf = torch.empty((num_blocks, num_kv_heads, rk + rv), dtype=dtype, device=device)
        return side_by_side(buf, rk)
    return (torch.empty((num_blocks, num_kv_heads, block_size, head_dim), dtype=dtype,
                        device=device),
            torch.empty((num_blocks, num_kv_heads, head_dim, block_size), dtype=dtype,
                        device=device))


def _dev(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _is_side_by_side(k_pool: torch.Tensor, v_pool: torch.Tensor) -> bool:
    """k_pool / v_pool are the K and V views of one side-by-side 8-bit
    buffer (see side_by_side)."""
    if k_pool.dtype != torch.uint8 or k_pool.dim() != 3 or v_pool.dim() != 3:
        return False
    nb, h, rk = k_pool.shape
    r = rk + v_pool.shape[2]
    want = (h * r, r, 1)
    return (k_pool.stride() == want and v_pool.stride() == want and
            v_pool.data_ptr() == k_pool.data_ptr() + rk and
            tuple(v_pool.shape[:2]) == (nb, h))


def _pools(k_pool: torch.Tensor, v_pool: torch.Tensor):
    """Device pointers of a pool pair: two contiguous buffers, or the views
    of one side-by-side 8-bit buffer."""
    if _is_side_by_side(k_pool, v_pool) and k_pool.is_cuda:
        return ctypes.c_void_p(k_pool.data_ptr()), ctypes.c_void_p(v_pool.data_ptr())
    return _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def pool_desc(k_pool: torch.Tensor, v_pool: torch.Tensor) -> PoolDesc:
    if k_pool.dtype == torch.uint8:
        if k_pool.dim() != 3 or v_pool.dim() != 3 or v_pool.dtype != torch.uint8:
            raise ValueError("8-bit pools must be uint8 [num_blocks][num_kv_heads][R]")
        nb, nkv, rk = k_pool.shape
        rv = v_pool.shape[2]
        if tuple(v_pool.shape[:2]) != (nb, nkv) or rk <= rv or (rk - rv) % 16:
            raise ValueError(f"8-bit regions of {rk} (K) and {rv} (V) bytes do not pair up: "
                             "R_k = B*(d+4), R_v = B*d with B a multiple of 4")
        B = (rk - rv) // 4
        if rv % B:
            raise ValueError(f"8-bit V region of {rv} bytes is not block_size * head_dim")
        return PoolDesc(nb, B, nkv, rv // B, PA_FP8_E4M3)
    if k_pool.dim() != 4:
        raise ValueError("k_pool must be [num_blocks][num_kv_heads][block_size][head_dim]")
    nb, nkv, B, d = k_pool.shape
    if tuple(v_pool.shape) != (nb, nkv, d, B) or v_pool.dtype != k_pool.dtype:
        raise ValueError("v_pool must be [num_blocks][num_kv_heads][head_dim][block_size] "
                         "with k_pool's dtype")
    return PoolDesc(nb, B, nkv, d, _dtype_code(k_pool))


def pa_kv_write(k_pool, v_pool, k_new, v_new, slot_mapping, stream=None):
    """Write each new token's K/V rows into its slot (negative slot: skip)."""
    desc = pool_desc(k_pool, v_pool)
    T = slot_mapping.numel()
    if slot_mapping.dtype != torch.int64:
        raise TypeError("slot_mapping must be int64")
    shape = (T, desc.num_kv_heads, desc.head_dim)
    if tuple(k_new.shape) != shape or tuple(v_new.shape) != shape:
        raise ValueError(f"k_new and v_new must be {shape}")
    if k_new.dtype != io_dtype(k_pool) or v_new.dtype != io_dtype(k_pool):
        raise TypeError("k_new/v_new must have the pool's element type (bf16 for 8-bit)")
    if T == 0:
        return
    st = _lib.pa_kv_write(ctypes.byref(desc), *_pools(k_pool, v_pool),
                          _dev(k_new, "k_new"), _dev(v_new, "v_new"),
                          _dev(slot_mapping, "slot_mapping"), T, _stream(stream))
    _check(st, "pa_kv_write")


def pa_decode_workspace_bytes(k_pool, v_pool, num_seqs, num_q_heads, max_blocks_per_seq,
                              partition_tokens=0):
    desc = pool_desc(k_pool, v_pool)
    return int(_lib.pa_decode_workspace_bytes(ctypes.byref(desc), num_seqs, num_q_heads,
                                              max_blocks_per_seq, partition_tokens))


def pa_decode_shared_workspace_bytes(k_pool, v_pool, num_seqs, num_q_heads,
                                     max_blocks_per_seq, partition_tokens=0):
    desc = pool_desc(k_pool, v_pool)
    return int(_lib.pa_decode_shared_workspace_bytes(ctypes.byref(desc), num_seqs, num_q_heads,
                                                     max_blocks_per_seq, partition_tokens))


def pa_decode_piece_tokens(k_pool, v_pool, num_seqs, num_q_heads, max_blocks_per_seq,
                           total_blocks, partition_tokens=0):
    """Length of the ranges pa_decode cuts a batch of total_blocks blocks into."""
    desc = pool_desc(k_pool, v_pool)
    return int(_lib.pa_decode_piece_tokens(ctypes.byref(desc), num_seqs, num_q_heads,
                                           max_blocks_per_seq, partition_tokens,
                                           int(total_blocks)))


def pa_decode_partition_tokens(k_pool, v_pool, num_seqs, num_q_heads, max_blocks_per_seq,
                               partition_tokens=0):
    desc = pool_desc(k_pool, v_pool)
    return int(_lib.pa_decode_partition_tokens(ctypes.byref(desc), num_seqs, num_q_heads,
                                               max_blocks_per_seq, partition_tokens))


def _decode_args(q, k_pool, v_pool, block_tables, context_lens, out):
    S, Hq, d = q.shape
    desc = pool_desc(k_pool, v_pool)
    if d != desc.head_dim or q.dtype != io_dtype(k_pool):
        raise ValueError("q must be [S][Hq][head_dim] in the pool's element type")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables must be [S][max_blocks] and context_lens [S]")
    if out is None:
        out = torch.empty_like(q)
    elif tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype:
        raise ValueError("out must match q")
    return desc, S, Hq, block_tables.shape[1], out


def _workspace(desc, S, Hq, maxB, partition_tokens, workspace, device, shared=False):
    query = _lib.pa_decode_shared_workspace_bytes if shared else _lib.pa_decode_workspace_bytes
    need = int(query(ctypes.byref(desc), S, Hq, maxB, partition_tokens))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else ctypes.c_void_p(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return ws_ptr, ws_bytes


def pa_decode(q, k_pool, v_pool, block_tables, context_lens, scale, out=None,
              partition_tokens=0, workspace=None, stream=None):
    """Paged decode attention; returns ``out`` [num_seqs][num_q_heads][head_dim].

    ``workspace`` is a uint8 GPU tensor of at least pa_decode_workspace_bytes
    bytes; when None one is allocated here with torch (the library itself
    never allocates)."""
    desc, S, Hq, maxB, out = _decode_args(q, k_pool, v_pool, block_tables, context_lens, out)
    ws_ptr, ws_bytes = _workspace(desc, S, Hq, maxB, partition_tokens, workspace, q.device)
    st = _lib.pa_decode(ctypes.byref(desc), *_pools(k_pool, v_pool),
                        _dev(q, "q"), S, Hq, _dev(block_tables, "block_tables"), maxB,
                        _dev(context_lens, "context_lens"), float(scale), _dev(out, "out"),
                        int(partition_tokens), ws_ptr, ws_bytes, _stream(stream))
    _check(st, "pa_decode")
    return out


def pa_decode_shared(q, k_pool, v_pool, block_tables, context_lens, scale, group_start,
                     shared_blocks, out=None, partition_tokens=0, workspace=None, stream=None):
    """pa_decode over prefix groups (int32 GPU tensors ``group_start``
    [G+1] and ``shared_blocks`` [G], e.g. from BlockManager.prefix_groups):
    each group's shared blocks are read once for all of its members."""
    desc, S, Hq, maxB, out = _decode_args(q, k_pool, v_pool, block_tables, context_lens, out)
    if group_start.dtype != torch.int32 or shared_blocks.dtype != torch.int32:
        raise TypeError("group_start and shared_blocks must be int32")
    n = shared_blocks.numel()
    if group_start.numel() != n + 1:
        raise ValueError("group_start must have one entry more than shared_blocks")
    ws_ptr, ws_bytes = _workspace(desc, S, Hq, maxB, partition_tokens, workspace, q.device,
                                  shared=n > 0)
    st = _lib.pa_decode_shared(
        ctypes.byref(desc), *_pools(k_pool, v_pool), _dev(q, "q"), S, Hq,
        _dev(block_tables, "block_tables"), maxB, _dev(context_lens, "context_lens"),
        float(scale), _dev(out, "out"), int(partition_tokens), n,
        _dev(group_start, "group_start") if n else ctypes.c_void_p(0),
        _dev(shared_blocks, "shared_blocks") if n else ctypes.c_void_p(0),
        ws_ptr, ws_bytes, _stream(stream))
    _check(st, "pa_decode_shared")
    return out


def pa_decode_step(q, k_pool, v_pool, k_new, v_new, block_tables, lens_in, lens_out,
                   new_blocks, scale, out=None, group_start=None, shared_blocks=None,
                   partition_tokens=0, workspace=None, stream=None):
    """One decode step: store each sequence's new token (k_new/v_new
    [S][Hkv][d] at position lens_in[s], in block new_blocks[s] or the
    table's tail block when -1), grow the tables, write lens_out = lens_in
    + 1 and decode over the grown contexts.  new_blocks: int32 [S] on the
    host (a numpy array or CPU tensor), read during the call."""
    desc, S, Hq, maxB, out = _decode_args(q, k_pool, v_pool, block_tables, lens_in, out)
    shape = (S, desc.num_kv_heads, desc.head_dim)
    if tuple(k_new.shape) != shape or tuple(v_new.shape) != shape:
        raise ValueError(f"k_new and v_new must be {shape}")
    if k_new.dtype != q.dtype or v_new.dtype != q.dtype:
        raise TypeError("k_new/v_new must be bf16")
    if lens_out.dtype != torch.int32 or lens_out.numel() != S or not lens_out.is_contiguous():
        raise ValueError("lens_out must be int32 [S], contiguous")
    nb_host = np.ascontiguousarray(np.asarray(new_blocks, dtype=np.int32).reshape(-1))
    if nb_host.size != S:
        raise ValueError("new_blocks must have one entry per sequence")
    nb_ptr = nb_host.ctypes.data_as(ctypes.c_void_p)
    n = 0 if shared_blocks is None else shared_blocks.numel()
    ws_ptr, ws_bytes = _workspace(desc, S, Hq, maxB, partition_tokens, workspace, q.device,
                                  shared=n > 0)
    st = _lib.pa_decode_step(
        ctypes.byref(desc), *_pools(k_pool, v_pool), _dev(q, "q"),
        _dev(k_new, "k_new"), _dev(v_new, "v_new"), S, Hq, _dev(block_tables, "block_tables"),
        maxB, _dev(lens_in, "lens_in"), _dev(lens_out, "lens_out"), nb_ptr, float(scale),
        _dev(out, "out"), int(partition_tokens), n,
        _dev(group_start, "group_start") if n else ctypes.c_void_p(0),
        _dev(shared_blocks, "shared_blocks") if n else ctypes.c_void_p(0),
        ws_ptr, ws_bytes, _stream(stream))
    _check(st, "pa_decode_step")
    return out


def pa_decode_noalloc(q, k_pool, v_pool, block_tables, context_lens, scale, out,
                      partition_tokens=0, stream=None):
    """pa_decode on the library's fixed device scratch: allocates nothing
    (``out`` must be given).  Calls that overlap on one GPU race."""
    if out is None:
        raise ValueError("pa_decode_noalloc needs out (it allocates nothing)")
    desc, S, Hq, maxB, out = _decode_args(q, k_pool, v_pool, block_tables, context_lens, out)
    st = _lib.pa_decode_noalloc(ctypes.byref(desc), *_pools(k_pool, v_pool), _dev(q, "q"), S, Hq,
                                _dev(block_tables, "block_tables"), maxB,
                                _dev(context_lens, "context_lens"), float(scale),
                                _dev(out, "out"), int(partition_tokens), _stream(stream))
    _check(st, "pa_decode_noalloc")
    return out


def pa_decode_noalloc_max_bytes():
    return int(_lib.pa_decode_noalloc_max_bytes())


def pa_extend_workspace_bytes(k_pool, v_pool, total_q, num_seqs, num_q_heads, max_blocks_per_seq):
    desc = pool_desc(k_pool, v_pool)
    return int(_lib.pa_extend_workspace_bytes(ctypes.byref(desc), total_q, num_seqs, num_q_heads,
                                              max_blocks_per_seq))


def pa_extend(q, k_pool, v_pool, q_start, block_tables, context_lens, scale, out=None,
              workspace=None, stream=None):
    """Multi-token causal attention (extend / chunked prefill); returns out
    [total_q][num_q_heads][head_dim].  Query j of sequence s (rows
    q_start[s] .. q_start[s+1]) sits at position context_lens[s] - n_s + j
    and attends to the sequence's tokens up to it."""
    desc = pool_desc(k_pool, v_pool)
    T, Hq, d = q.shape
    if d != desc.head_dim or q.dtype != io_dtype(k_pool):
        raise ValueError("q must be [total][Hq][head_dim] in the pool's element type")
    for t, name in ((q_start, "q_start"), (block_tables, "block_tables"),
                    (context_lens, "context_lens")):
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32")
    S = context_lens.numel()
    if q_start.numel() != S + 1 or block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("q_start must be [S+1] and block_tables [S][max_blocks]")
    if out is None:
        out = torch.empty_like(q)
    elif tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if workspace is None:
        need = int(_lib.pa_extend_workspace_bytes(ctypes.byref(desc), T, S, Hq,
                                                  block_tables.shape[1])) if T and S else 0
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else ctypes.c_void_p(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _lib.pa_extend(ctypes.byref(desc), *_pools(k_pool, v_pool),
                        _dev(q, "q"), T, _dev(q_start, "q_start"), S, Hq,
                        _dev(block_tables, "block_tables"), block_tables.shape[1],
                        _dev(context_lens, "context_lens"), float(scale), _dev(out, "out"),
                        ws_ptr, ws_bytes, _stream(stream))
    _check(st, "pa_extend")
    return out


def pa_block_copy(k_pool, v_pool, pairs, stream=None):
    """Copy whole blocks (every kv head and slot) for each (src, dst) pair."""
    desc = pool_desc(k_pool, v_pool)
    if pairs.dtype != torch.int32 or (pairs.numel() and pairs.shape[-1] != 2):
        raise ValueError("pairs must be int32 [P][2]")
    n = pairs.numel() // 2
    if n == 0:
        return
    st = _lib.pa_block_copy(ctypes.byref(desc), *_pools(k_pool, v_pool),
                            _dev(pairs, "pairs"), n, _stream(stream))
    _check(st, "pa_block_copy")


def alloc_host_pools(num_host_blocks, k_pool, v_pool):
    """Pinned host pools of num_host_blocks blocks with k_pool / v_pool's
    per-block layout (swap space for pa_block_swap); side-by-side 8-bit
    pools get a side-by-side host buffer."""
    if _is_side_by_side(k_pool, v_pool):
        buf = torch.empty((num_host_blocks, k_pool.shape[1], k_pool.shape[2] + v_pool.shape[2]),
                          dtype=torch.uint8, pin_memory=True)
        return side_by_side(buf, k_pool.shape[2])
    return (torch.empty((num_host_blocks,) + tuple(k_pool.shape[1:]), dtype=k_pool.dtype,
                        pin_memory=True),
            torch.empty((num_host_blocks,) + tuple(v_pool.shape[1:]), dtype=v_pool.dtype,
                        pin_memory=True))


def pa_block_swap(k_pool, v_pool, host_k, host_v, pairs, direction, stream=None):
    """Move whole blocks between the device pools and pinned host pools:
    PA_SWAP_OUT copies device block src to host block dst, PA_SWAP_IN host
    block src to device block dst, for each (src, dst) row of ``pairs``."""
    desc = pool_desc(k_pool, v_pool)
    sbs = _is_side_by_side(k_pool, v_pool)
    if sbs != _is_side_by_side(host_k, host_v):
        raise ValueError("host_k / host_v must share the pools' layout (side-by-side 8-bit "
                         "regions or two buffers)")
    for t, pool, name in ((host_k, k_pool, "host_k"), (host_v, v_pool, "host_v")):
        if not isinstance(t, torch.Tensor) or t.is_cuda or not t.is_pinned():
            raise TypeError(f"{name} must be a pinned host tensor")
        if not (sbs or t.is_contiguous()) or t.dtype != pool.dtype or \
                tuple(t.shape[1:]) != tuple(pool.shape[1:]):
            raise ValueError(f"{name} must be contiguous with the pool's block layout")
    if host_k.shape[0] != host_v.shape[0]:
        raise ValueError("host_k and host_v must hold the same number of blocks")
    if pairs.dtype != torch.int32 or (pairs.numel() and pairs.shape[-1] != 2):
        raise ValueError("pairs must be int32 [P][2]")
    n = pairs.numel() // 2
    if n == 0:
        return
    st = _lib.pa_block_swap(ctypes.byref(desc), *_pools(k_pool, v_pool),
                            ctypes.c_void_p(host_k.data_ptr()), ctypes.c_void_p(host_v.data_ptr()),
                            int(host_k.shape[0]), _dev(pairs, "pairs"), n, int(direction),
                            _stream(stream))
    _check(st, "pa_block_swap")


def pa_table_update(block_tables, block_size, seq_ids, positions, slot_mapping, stream=None):
    """Point each written token's table entry at the block it was written to."""
    T = slot_mapping.numel()
    if seq_ids.dtype != torch.int32 or positions.dtype != torch.int32 or \
            slot_mapping.dtype != torch.int64 or block_tables.dtype != torch.int32:
        raise TypeError("block_tables/seq_ids/positions int32, slot_mapping int64")
    if seq_ids.numel() != T or positions.numel() != T:
        raise ValueError("seq_ids, positions and slot_mapping must have one entry per token")
    if T == 0:
        return
    st = _lib.pa_table_update(_dev(block_tables, "block_tables"), block_tables.shape[1],
                              int(block_size), _dev(seq_ids, "seq_ids"),
                              _dev(positions, "positions"), _dev(slot_mapping, "slot_mapping"),
                              T, _stream(stream))
    _check(st, "pa_table_update")


def pa_kv_append(k_pool, v_pool, k_new, v_new, slot_mapping, block_tables, seq_ids, positions,
                 stream=None):
    """pa_table_update and pa_kv_write in one launch."""
    desc = pool_desc(k_pool, v_pool)
    T = slot_mapping.numel()
    if slot_mapping.dtype != torch.int64 or seq_ids.dtype != torch.int32 or \
            positions.dtype != torch.int32 or block_tables.dtype != torch.int32:
        raise TypeError("block_tables/seq_ids/positions int32, slot_mapping int64")
    shape = (T, desc.num_kv_heads, desc.head_dim)
    if tuple(k_new.shape) != shape or tuple(v_new.shape) != shape:
        raise ValueError(f"k_new and v_new must be {shape}")
    if k_new.dtype != io_dtype(k_pool) or v_new.dtype != io_dtype(k_pool):
        raise TypeError("k_new/v_new must have the pool's element type (bf16 for 8-bit)")
    if seq_ids.numel() != T or positions.numel() != T:
        raise ValueError("seq_ids, positions and slot_mapping must have one entry per token")
    if T == 0:
        return
    st = _lib.pa_kv_append(ctypes.byref(desc), *_pools(k_pool, v_pool),
                           _dev(k_new, "k_new"), _dev(v_new, "v_new"),
                           _dev(slot_mapping, "slot_mapping"), T,
                           _dev(block_tables, "block_tables"), block_tables.shape[1],
                           _dev(seq_ids, "seq_ids"), _dev(positions, "positions"),
                           _stream(stream))
    _check(st, "pa_kv_append")


def pa_probe_read(buf, order, chunk_bytes, workgroups, loads_in_flight=4, sink=None,
                  stream=None):
    """Read buf's chunks in the given order (pa_probe_read); returns sink."""
    if order.dtype != torch.int32:
        raise TypeError("order must be int32")
    need = int(_lib.pa_probe_sink_bytes(int(workgroups)))
    if sink is None:
        sink = torch.empty(need, dtype=torch.uint8, device=buf.device)
    if sink.numel() * sink.element_size() < need:
        raise ValueError("sink too small")
    n = order.numel()
    if n * int(chunk_bytes) > buf.numel() * buf.element_size():
        raise ValueError("chunks reach past the buffer")
    if n and int(order.max()) * int(chunk_bytes) + int(chunk_bytes) > buf.numel() * buf.element_size():
        raise ValueError("a chunk index reaches past the buffer")
    st = _lib.pa_probe_read(_dev(buf, "buf"), _dev(order, "order"), n, int(chunk_bytes),
                            int(workgroups), int(loads_in_flight), _dev(sink, "sink"),
                            _stream(stream))
    _check(st, "pa_probe_read")
    return sink


from .block_manager import BlockManager  # noqa: E402,F401
