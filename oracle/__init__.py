"""CPU oracle for paged decode attention, slot writes, block copies and the
host block manager.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The product (the HIP library and
its Python binding) never imports it, and the two share no code: the only
thing both sides consume is the seeded input data produced by ``workloads``.

The numeric oracle is plain C (``oracle.c``) working in double; this module
is the ctypes marshalling around it.  ``bm_model`` is the block-manager
reference model, in Python.
"""
import ctypes
import os

import numpy as np

from .build import LIB, build

F32 = 0
BF16 = 1
FP8 = 2

_lib = None


def lib():
    """Load liboracle.so, building it with gcc first if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        i32, f64, vp = ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        L.oracle_decode_pairs.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, i32, i32,
                                          vp, i32, vp, f64, vp, i32, vp, i32]
        L.oracle_decode.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, i32, i32, vp,
                                    i32, vp, f64, vp, i32]
        L.oracle_decode_dense.argtypes = [i32, i32, i32, vp, vp, i32, vp, i32, i32, vp,
                                          f64, vp, i32]
        L.oracle_decode_split.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, i32, i32,
                                          vp, i32, vp, f64, i32, vp, i32]
        L.oracle_gather.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, i32, i32, i32,
                                    vp, vp]
        L.oracle_kv_write.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, i32]
        L.oracle_block_copy.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, i32]
        L.oracle_max_threads.argtypes = []
        L.oracle_extend.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, i32, i32, vp, i32,
                                    vp, f64, vp, i32]
        L.oracle_extend.restype = ctypes.c_int
        L.oracle_block_swap.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, i32, vp, i32,
                                        i32]
        L.oracle_block_swap.restype = ctypes.c_int
        L.oracle_e4m3_encode.argtypes = [vp, vp, i32]
        L.oracle_e4m3_decode.argtypes = [vp, vp, i32]
        L.oracle_e4m3_encode.restype = None
        L.oracle_e4m3_decode.restype = None
        for fn in ("oracle_decode_pairs", "oracle_decode", "oracle_decode_dense",
                   "oracle_decode_split", "oracle_gather", "oracle_kv_write",
                   "oracle_block_copy", "oracle_max_threads"):
            getattr(L, fn).restype = ctypes.c_int
        _lib = L
    return _lib


def _dtype_code(arr):
    if arr.dtype == np.float32:
        return F32
    if arr.dtype == np.uint16:  # bf16 bit patterns
        return BF16
    if arr.dtype == np.uint8:  # 8-bit regions: E4M3 codes (K: then per-token bf16 scales)
        return FP8
    raise TypeError(f"pool dtype must be float32, uint16 (bf16 bits) or uint8 (8-bit "
                    f"regions), got {arr.dtype}")


def _c(arr, dtype=None):
    a = np.ascontiguousarray(arr if dtype is None else arr.astype(dtype, copy=False))
    return a, a.ctypes.data_as(ctypes.c_void_p)


class OracleError(RuntimeError):
    pass


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what} failed with code {rc}")


def fp8_region_bytes(block_size, head_dim):
    """Bytes of one (block, kv head) region of an 8-bit pool: (K buffer, V
    buffer).  K: block_size * head_dim E4M3 codes (token-major [B][d]), then
    the bf16 scales of the region's slots, per group of 4 slots its 4 K
    scales then its 4 V scales.  V: block_size * head_dim codes (dim-major
    [d][B])."""
    return block_size * head_dim + 4 * block_size, block_size * head_dim


def _geom(k_pool, v_pool):
    """(num_blocks, B, H_kv, d) of a pool pair.  fp32 / bf16 pools are
    [num_blocks][H_kv][B][d] and [num_blocks][H_kv][d][B]; 8-bit pools are
    uint8 [num_blocks][H_kv][B*(d+4)] and [num_blocks][H_kv][B*d]."""
    if k_pool.dtype == np.uint8:
        nb, nkv, rk = k_pool.shape
        rv = v_pool.shape[2]
        if v_pool.shape[:2] != (nb, nkv) or rk <= rv or (rk - rv) % 4:
            raise ValueError(f"8-bit regions of {rk} and {rv} bytes do not pair up")
        B = (rk - rv) // 4
        if rv % B:
            raise ValueError(f"8-bit V region of {rv} bytes is not B * d for B = {B}")
        return nb, B, nkv, rv // B
    nb, nkv, B, d = k_pool.shape
    return nb, B, nkv, d


def decode(k_pool, v_pool, q, block_tables, context_lens, scale, threads=0):
    """Paged decode attention for every (sequence, query head).

    k_pool [nb][Hkv][B][d], v_pool [nb][Hkv][d][B], q [S][Hq][d]: float32 or
    uint16 holding bf16 bits.  block_tables int32 [S][maxB], context_lens int32
    [S].  Returns float64 [S][Hq][d].
    """
    S, Hq, _ = q.shape
    nb, B, nkv, d = _geom(k_pool, v_pool)
    kp, kpp = _c(k_pool)
    vp_, vpp = _c(v_pool)
    qq, qp = _c(q)
    bt, btp = _c(block_tables, np.int32)
    cl, clp = _c(context_lens, np.int32)
    out = np.empty((S, Hq, d), np.float64)
    rc = lib().oracle_decode(_dtype_code(k_pool), nb, B, nkv, d, kpp, vpp, qp, S, Hq,
                             btp, bt.shape[1], clp, float(scale),
                             out.ctypes.data_as(ctypes.c_void_p), int(threads))
    _check(rc, "oracle_decode")
    return out


def decode_pairs(k_pool, v_pool, q, block_tables, context_lens, scale, pairs, threads=0):
    """Paged decode attention for selected (sequence, query head) pairs.
    Returns float64 [n_pairs][d]."""
    S, Hq, _ = q.shape
    nb, B, nkv, d = _geom(k_pool, v_pool)
    kp, kpp = _c(k_pool)
    vp_, vpp = _c(v_pool)
    qq, qp = _c(q)
    bt, btp = _c(block_tables, np.int32)
    cl, clp = _c(context_lens, np.int32)
    pr, prp = _c(np.asarray(pairs).reshape(-1, 2), np.int32)
    out = np.empty((pr.shape[0], d), np.float64)
    rc = lib().oracle_decode_pairs(_dtype_code(k_pool), nb, B, nkv, d, kpp, vpp, qp, S,
                                   Hq, btp, bt.shape[1], clp, float(scale), prp,
                                   pr.shape[0], out.ctypes.data_as(ctypes.c_void_p),
                                   int(threads))
    _check(rc, "oracle_decode_pairs")
    return out


def decode_dense(k_dense, v_dense, q, context_lens, scale, threads=0):
    """Unpaged attention: k_dense, v_dense [S][Hkv][max_len][d] (token-major).
    Returns float64 [S][Hq][d]."""
    S, nkv, max_len, d = k_dense.shape
    _, Hq, _ = q.shape
    kd, kdp = _c(k_dense)
    vd, vdp = _c(v_dense)
    qq, qp = _c(q)
    cl, clp = _c(context_lens, np.int32)
    out = np.empty((S, Hq, d), np.float64)
    rc = lib().oracle_decode_dense(_dtype_code(k_dense), nkv, d, kdp, vdp, max_len, qp,
                                   S, Hq, clp, float(scale),
                                   out.ctypes.data_as(ctypes.c_void_p), int(threads))
    _check(rc, "oracle_decode_dense")
    return out


def decode_split(k_pool, v_pool, q, block_tables, context_lens, scale, partition_tokens,
                 threads=0):
    """Split-context attention (partials combined by max/sum-exp)."""
    S, Hq, _ = q.shape
    nb, B, nkv, d = _geom(k_pool, v_pool)
    kp, kpp = _c(k_pool)
    vp_, vpp = _c(v_pool)
    qq, qp = _c(q)
    bt, btp = _c(block_tables, np.int32)
    cl, clp = _c(context_lens, np.int32)
    out = np.empty((S, Hq, d), np.float64)
    rc = lib().oracle_decode_split(_dtype_code(k_pool), nb, B, nkv, d, kpp, vpp, qp, S,
                                   Hq, btp, bt.shape[1], clp, float(scale),
                                   int(partition_tokens),
                                   out.ctypes.data_as(ctypes.c_void_p), int(threads))
    _check(rc, "oracle_decode_split")
    return out


def gather(k_pool, v_pool, table_row, kv_head, length):
    """Walk one table row and return contiguous float64 (Kc [L][d], Vc [L][d]),
    dequantised for 8-bit pools."""
    nb, B, nkv, d = _geom(k_pool, v_pool)
    kp, kpp = _c(k_pool)
    vp_, vpp = _c(v_pool)
    tr, trp = _c(table_row, np.int32)
    Kc = np.empty((length, d), np.float64)
    Vc = np.empty((length, d), np.float64)
    rc = lib().oracle_gather(_dtype_code(k_pool), nb, B, nkv, d, kpp, vpp, trp,
                             tr.shape[0], int(kv_head), int(length),
                             Kc.ctypes.data_as(ctypes.c_void_p),
                             Vc.ctypes.data_as(ctypes.c_void_p))
    _check(rc, "oracle_gather")
    return Kc, Vc


def kv_write(k_pool, v_pool, k_new, v_new, slot_mapping):
    """Return copies of the pools with each token's K/V written into its slot.
    k_new, v_new [T][H_kv][d] have the pool's element type, or bf16 bits
    (uint16) for an 8-bit pool, which stores them quantised."""
    nb, B, nkv, d = _geom(k_pool, v_pool)
    kp = np.array(k_pool, copy=True, order="C")
    vp_ = np.array(v_pool, copy=True, order="C")
    src_dtype = np.uint16 if kp.dtype == np.uint8 else kp.dtype
    kn, knp = _c(k_new, src_dtype)
    vn, vnp = _c(v_new, src_dtype)
    sm, smp = _c(slot_mapping, np.int64)
    rc = lib().oracle_kv_write(_dtype_code(kp), nb, B, nkv, d,
                               kp.ctypes.data_as(ctypes.c_void_p),
                               vp_.ctypes.data_as(ctypes.c_void_p), knp, vnp, smp,
                               sm.shape[0])
    _check(rc, "oracle_kv_write")
    return kp, vp_


def block_copy(k_pool, v_pool, pairs):
    """Return copies of the pools with each (src, dst) block copied."""
    nb, B, nkv, d = _geom(k_pool, v_pool)
    kp = np.array(k_pool, copy=True, order="C")
    vp_ = np.array(v_pool, copy=True, order="C")
    pr, prp = _c(np.asarray(pairs).reshape(-1, 2), np.int32)
    rc = lib().oracle_block_copy(_dtype_code(kp), nb, B, nkv, d,
                                 kp.ctypes.data_as(ctypes.c_void_p),
                                 vp_.ctypes.data_as(ctypes.c_void_p), prp, pr.shape[0])
    _check(rc, "oracle_block_copy")
    return kp, vp_


def extend(k_pool, v_pool, q, q_start, block_tables, context_lens, scale, threads=0):
    """Multi-token causal attention: q [total][Hq][d] rows of the sequences
    given by q_start [S+1]; query j of sequence s sits at position
    context_lens[s] - n_s + j and attends to tokens 0..that position.
    Returns float64 [total][Hq][d]."""
    nb, B, nkv, d = _geom(k_pool, v_pool)
    T, Hq, _ = q.shape
    kp, kpp = _c(k_pool)
    vp_, vpp = _c(v_pool)
    qq, qp = _c(q)
    qs, qsp = _c(q_start, np.int32)
    bt, btp = _c(block_tables, np.int32)
    cl, clp = _c(context_lens, np.int32)
    if qs[-1] != T:
        raise ValueError("q_start[-1] must equal the number of query rows")
    out = np.empty((T, Hq, d), np.float64)
    rc = lib().oracle_extend(_dtype_code(k_pool), nb, B, nkv, d, kpp, vpp, qp, qsp,
                             len(qs) - 1, Hq, btp, bt.shape[1], clp, float(scale),
                             out.ctypes.data_as(ctypes.c_void_p), int(threads))
    _check(rc, "oracle_extend")
    return out


SWAP_OUT, SWAP_IN = 0, 1


def block_swap(k_pool, v_pool, host_k, host_v, pairs, direction):
    """Return copies (k_pool, v_pool, host_k, host_v) after moving each
    (src, dst) block: device -> host for SWAP_OUT, host -> device for SWAP_IN.
    Host pools have the device pools' per-block layout."""
    nb, B, nkv, d = _geom(k_pool, v_pool)
    kp = np.array(k_pool, copy=True, order="C")
    vp_ = np.array(v_pool, copy=True, order="C")
    hk = np.array(host_k, copy=True, order="C")
    hv = np.array(host_v, copy=True, order="C")
    if hk.shape[1:] != kp.shape[1:] or hv.shape[1:] != vp_.shape[1:] or hk.dtype != kp.dtype:
        raise ValueError("host pools must have the device pools' block layout")
    pr, prp = _c(np.asarray(pairs).reshape(-1, 2), np.int32)
    rc = lib().oracle_block_swap(_dtype_code(kp), nb, B, nkv, d,
                                 kp.ctypes.data_as(ctypes.c_void_p),
                                 vp_.ctypes.data_as(ctypes.c_void_p),
                                 hk.ctypes.data_as(ctypes.c_void_p),
                                 hv.ctypes.data_as(ctypes.c_void_p), hk.shape[0], prp,
                                 pr.shape[0], int(direction))
    _check(rc, "oracle_block_swap")
    return kp, vp_, hk, hv


def e4m3_encode(x):
    """OCP E4M3 codes (uint8) of float32 values, nearest even, saturating."""
    xx, xp = _c(np.asarray(x, np.float32).reshape(-1), np.float32)
    out = np.empty(xx.shape[0], np.uint8)
    lib().oracle_e4m3_encode(xp, out.ctypes.data_as(ctypes.c_void_p), xx.shape[0])
    return out.reshape(np.shape(x))


def e4m3_decode(codes):
    """Values (float64) of OCP E4M3 codes; NaN for the two NaN codes."""
    cc, cp = _c(np.asarray(codes, np.uint8).reshape(-1), np.uint8)
    out = np.empty(cc.shape[0], np.float64)
    lib().oracle_e4m3_decode(cp, out.ctypes.data_as(ctypes.c_void_p), cc.shape[0])
    return out.reshape(np.shape(codes))


def max_threads():
    return int(lib().oracle_max_threads())
