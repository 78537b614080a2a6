"""GPU parity: the HIP path (through the C-ABI) against the CPU oracle on the
same seeded inputs.

Bars: slot writes, block copies, table updates and block-manager output
bit-exact; attention max |GPU - oracle| <= 2e-2 for bf16 storage and 1e-4
for fp32 (fp32 accumulation on the GPU, fp64 in the oracle).
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle.bm_model import BlockManagerModel
from workloads import (CONFIGS, POISON_V, block_copy_case, decode_case, kv_write_case)
from workloads.gen import fp8_poison, fp8_region_bytes, from_numpy_storage, to_numpy_storage

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def pk():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import paged_kv_cache_335_amd as pk
    return pk


def _gpu_decode(pk, c, partition_tokens=0):
    out = pk.pa_decode(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens, c.scale,
                       partition_tokens=partition_tokens)
    torch.cuda.synchronize()
    return out


def _to64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _check(got, ref, dtype, what):
    err = np.abs(got - ref)
    _log(f"{what}: max|err| {err.max():.3e} mean {err.mean():.3e}")
    assert np.isfinite(got).all(), what
    assert err.max() <= TOL[dtype], f"{what}: max err {err.max()}"


# --- reduced-size configs, every output element -----------------------------
SMALL = {
    "tiny_f32": CONFIGS["tiny_f32"],
    "llama2_7b_mha": CONFIGS["llama2_7b_mha"].scaled(num_seqs=6, lengths=("uniform", 128, 700), pool=("fixed", 512),
                                   table_width=48),
    "llama3_8b_gqa": CONFIGS["llama3_8b_gqa"].scaled(num_seqs=24, lengths=("lognormal", 256, 1.0, 16, 2048),
                                   table_width=128),
    "prefix_sharing": CONFIGS["prefix_sharing"].scaled(num_seqs=16, prompts=4, lengths=("shared", 96, 1, 40),
                                   table_width=9),
    "prefix_sharing_cow": CONFIGS["prefix_sharing_cow"].scaled(num_seqs=16, prompts=4, lengths=("shared", 104, 1, 40),
                                         table_width=10),
    "long_context_128k": CONFIGS["long_context_128k"].scaled(num_seqs=2, lengths=("fixed", 4096), pool=("fixed", 512),
                                   table_width=256),
}


@pytest.mark.parametrize("key", list(SMALL))
def test_decode_small_configs_all_elements(pk, key):
    cfg = SMALL[key]
    c = decode_case(cfg, payload="numpy", device="cuda")
    ref = oracle.decode(*c.oracle_inputs(), c.scale)
    parts = [0, cfg.partition_tokens or 64, 16]
    for P in parts:
        got = _to64(_gpu_decode(pk, c, P))
        _check(got, ref, cfg.dtype, f"{key} P={P}")


def _custom_case(lens, Hq, Hkv, d, nb, width, seed, dtype="bf16"):
    """Random pools (no poison) and independent random tables per sequence
    (rows may share blocks: decode only reads)."""
    from types import SimpleNamespace
    rng = np.random.default_rng(seed)
    S, B = len(lens), 16
    tables = np.stack([rng.permutation(nb)[:width] for _ in lens]).astype(np.int32)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = torch.from_numpy(rng.standard_normal((S, Hq, d), dtype=np.float32)).to(tdt)
    k = torch.from_numpy(rng.standard_normal((nb, Hkv, B, d), dtype=np.float32)).to(tdt)
    v = torch.from_numpy(rng.standard_normal((nb, Hkv, d, B), dtype=np.float32)).to(tdt)
    lens = np.asarray(lens, np.int32)
    c = SimpleNamespace(q=q.cuda(), k_pool=k.cuda(), v_pool=v.cuda(),
                        block_tables=torch.from_numpy(tables).cuda(),
                        context_lens=torch.from_numpy(lens).cuda(), scale=d ** -0.5)
    c.oracle_inputs = lambda: (to_numpy_storage(k), to_numpy_storage(v), to_numpy_storage(q),
                               tables, lens)
    return c


@pytest.mark.parametrize("G,d", [(1, 64), (1, 128), (2, 128), (3, 128), (4, 64), (4, 128),
                                 (5, 128), (8, 128), (16, 64), (16, 128)])
def test_decode_group_sizes_and_head_dims(pk, G, d):
    """Every kernel family and padding case: VALU (G <= 2) and MFMA
    (G 3..16), head dims 64 and 128, lengths around block and partition
    edges."""
    lens = (1, 15, 16, 17, 63, 64, 65, 511, 512, 513)
    c = _custom_case(lens, Hq=2 * G, Hkv=2, d=d, nb=300, width=40, seed=100 + G)
    ref = oracle.decode(*c.oracle_inputs(), c.scale)
    for P in (0, 64, 256):
        _check(_to64(_gpu_decode(pk, c, P)), ref, "bf16", f"G={G} d={d} P={P}")


@pytest.mark.parametrize("scale", [0.0, -0.3, 4.0])
def test_decode_extreme_scales(pk, scale):
    """Zero scale (plain mean of V), a negative scale, and a large one whose
    scores spread over dozens of log2 units, so the running reference moves
    often: MFMA kernel with 1 and 4 query heads per kv head, and the fp32
    VALU kernel, against the oracle."""
    lens = (1, 2, 15, 16, 17, 200, 513, 1000)
    for Hq, Hkv, dtype in ((8, 2, "bf16"), (2, 2, "bf16"), (4, 2, "f32")):
        c = _custom_case(lens, Hq=Hq, Hkv=Hkv, d=128, nb=300, width=63, seed=7, dtype=dtype)
        ref = oracle.decode(*c.oracle_inputs(), scale)
        out = pk.pa_decode(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens, scale)
        torch.cuda.synchronize()
        _check(_to64(out), ref, dtype, f"scale={scale} Hq={Hq} {dtype}")


@pytest.mark.parametrize("Hkv", [1, 3, 5, 6, 12])
def test_decode_kv_head_counts(pk, Hkv):
    """Kv-head counts that are not a multiple of a workgroup's four waves:
    the grid's waves take (kv head, range) pairs in turn, so a workgroup can
    mix heads and ranges.  MFMA and fp32 VALU kernels, two partition
    floors, every output against the oracle."""
    lens = (1, 16, 17, 100, 511, 1200)
    for G, dtype in ((2, "bf16"), (3, "f32")):
        c = _custom_case(lens, Hq=G * Hkv, Hkv=Hkv, d=64, nb=300, width=80, seed=500 + Hkv,
                         dtype=dtype)
        ref = oracle.decode(*c.oracle_inputs(), c.scale)
        for P in (0, 64):
            _check(_to64(_gpu_decode(pk, c, P)), ref, dtype, f"Hkv={Hkv} G={G} {dtype} P={P}")


def test_decode_fp32_group_sizes(pk):
    """fp32 pools, 1 to 16 query heads per kv head: above four the kernel
    takes the query heads in groups of 4, 3, 2 or 1 (the largest that
    divides G), each group a head of the plan over the same kv head."""
    for G in (1, 2, 4, 5, 6, 8, 9, 16):
        cfg = CONFIGS["tiny_f32"].scaled(num_seqs=5, num_q_heads=G, num_kv_heads=1, head_dim=128,
                                     lengths=("uniform", 1, 200), pool=("fixed", 80),
                                     table_width=16, seed=30 + G, key="f32g")
        c = decode_case(cfg, payload="numpy", device="cuda")
        ref = oracle.decode(*c.oracle_inputs(), c.scale)
        for P in (0, 32):
            _check(_to64(_gpu_decode(pk, c, P)), ref, "f32", f"fp32 G={G} P={P}")
    # several kv heads, each taken as head groups (6 = 2 groups of 3; 8 = 2 of
    # 4): the groups' pool offsets and query heads interleave per kv head
    for G, Hkv in ((6, 3), (8, 5)):
        c = _custom_case((1, 16, 17, 100, 511), Hq=G * Hkv, Hkv=Hkv, d=64, nb=200, width=40,
                         seed=540 + G, dtype="f32")
        ref = oracle.decode(*c.oracle_inputs(), c.scale)
        for P in (0, 64):
            _check(_to64(_gpu_decode(pk, c, P)), ref, "f32", f"fp32 Hkv={Hkv} G={G} P={P}")


def test_nan_in_unused_tail_slots_never_reaches_output(pk):
    cfg = SMALL["llama3_8b_gqa"]
    c = decode_case(cfg, payload="numpy", device="cuda")
    ref = oracle.decode(*c.oracle_inputs(), c.scale)
    dead = torch.from_numpy(~c.live).cuda()
    c.k_pool.masked_fill_(dead[:, None, :, None], float("nan"))
    c.v_pool.masked_fill_(dead[:, None, None, :], float("nan"))
    _check(_to64(_gpu_decode(pk, c, 0)), ref, "bf16", "nan tails")


def test_deterministic_and_placement_invariant(pk):
    """Same inputs twice: identical bits.  Same logical data moved to other
    physical blocks (tables renumbered): identical bits."""
    cfg = SMALL["llama3_8b_gqa"]
    c = decode_case(cfg, payload="numpy", device="cuda")
    a = _gpu_decode(pk, c, 64).clone()
    b = _gpu_decode(pk, c, 64)
    assert torch.equal(a, b)
    nb = c.num_blocks
    move = torch.from_numpy(np.random.default_rng(5).permutation(nb)).cuda()
    k2 = torch.empty_like(c.k_pool)
    v2 = torch.empty_like(c.v_pool)
    k2[move] = c.k_pool
    v2[move] = c.v_pool
    t2 = move[c.block_tables.long()].to(torch.int32).contiguous()
    out2 = pk.pa_decode(c.q, k2, v2, t2, c.context_lens, c.scale, partition_tokens=64)
    torch.cuda.synchronize()
    assert torch.equal(a, out2)


def test_decode_plan_equal_tail_buckets(pk):
    """Many sequences whose last partitions have the same length (the same
    bucket of the work plan), over several placement chunks and far more
    units than workgroups: every output against the oracle, and three calls
    bit-identical.  A plan that differed between workgroups would skip some
    units and repeat others."""
    rng = np.random.default_rng(77)
    S, P = 600, 64
    lens = 64 * rng.integers(0, 4, S) + rng.choice([5, 5, 5, 37, 64], S)
    c = _custom_case(lens, Hq=16, Hkv=4, d=64, nb=40, width=16, seed=78)
    ref = oracle.decode(*c.oracle_inputs(), c.scale)
    a = _gpu_decode(pk, c, P).clone()
    _check(_to64(a), ref, "bf16", "equal tails")
    for _ in range(2):
        assert torch.equal(a, _gpu_decode(pk, c, P))


def test_decode_batch_beyond_one_launch(pk):
    """More sequences than one launch plans for (the batch is split into
    slices): every output against the oracle, split and unsplit sequences."""
    rng = np.random.default_rng(91)
    lens = rng.integers(1, 101, 4100)
    c = _custom_case(lens, Hq=4, Hkv=1, d=64, nb=64, width=7, seed=92)
    ref = oracle.decode(*c.oracle_inputs(), c.scale)
    for P in (32, 0):
        _check(_to64(_gpu_decode(pk, c, P)), ref, "bf16", f"S=4100 P={P}")


def test_decode_short_tables_default_partition(pk):
    """Short tables take a floor below 256 tokens by default (one block for
    a 1- or 3-block table): hundreds of short sequences then spread over many
    ranges and are cut across range boundaries.  Every output against the
    oracle, with the library's choice and with an explicit 256."""
    rng = np.random.default_rng(93)
    for width, hi in ((1, 16), (3, 40)):
        lens = rng.integers(1, hi + 1, 600)
        c = _custom_case(lens, Hq=8, Hkv=2, d=128, nb=400, width=width, seed=94 + width)
        P0 = pk.pa_decode_partition_tokens(c.k_pool, c.v_pool, 600, 8, width)
        assert P0 == 16, P0
        ref = oracle.decode(*c.oracle_inputs(), c.scale)
        for P in (0, 256):
            _check(_to64(_gpu_decode(pk, c, P)), ref, "bf16", f"width={width} P={P}")


def test_pools_beyond_4_gib(pk):
    """Pools of 4.1 GiB each, every block the test touches above the 4 GiB
    mark (byte offsets past 2^32 in both pools): decode, extend, slot write
    and block copy against the oracle on compact host copies of the touched
    blocks."""
    Hkv, d, B, Hq = 8, 128, 16, 32
    blk = Hkv * B * d * 2                      # bytes of one block in each pool
    lo_n = (4 << 30) // blk                    # blocks below the 4 GiB mark
    nb = lo_n + 4096
    dev = torch.device("cuda")
    k = torch.empty((nb, Hkv, B, d), dtype=torch.bfloat16, device=dev)
    v = torch.empty((nb, Hkv, d, B), dtype=torch.bfloat16, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    k.normal_(generator=g)
    v.normal_(generator=g)
    rng = np.random.default_rng(8)
    hi = np.arange(lo_n, nb)

    def host(pool, ids):
        return to_numpy_storage(pool[torch.from_numpy(np.asarray(ids, np.int64)).to(dev)])

    # decode over tables of high blocks
    lens = np.array([1, 100, 777, 1500], np.int32)
    width = int((lens.max() + B - 1) // B)
    ids = rng.permutation(hi)[:len(lens) * width].reshape(len(lens), width).astype(np.int32)
    q = torch.randn((len(lens), Hq, d), generator=g, device=dev).to(torch.bfloat16)
    out = pk.pa_decode(q, k, v, torch.from_numpy(ids).to(dev), torch.from_numpy(lens).to(dev),
                       d ** -0.5)
    torch.cuda.synchronize()
    used = np.unique(ids)
    ref = oracle.decode(host(k, used), host(v, used), to_numpy_storage(q),
                        np.searchsorted(used, ids).astype(np.int32), lens, d ** -0.5)
    _check(_to64(out), ref, "bf16", "decode over blocks past 4 GiB")
    # extend (the last n tokens of each context as queries) over the same tables
    n = np.minimum(lens, 24).astype(np.int32)
    q_start = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    qe = torch.randn((int(q_start[-1]), Hq, d), generator=g, device=dev).to(torch.bfloat16)
    oute = pk.pa_extend(qe, k, v, torch.from_numpy(q_start).to(dev), torch.from_numpy(ids).to(dev),
                        torch.from_numpy(lens).to(dev), d ** -0.5)
    torch.cuda.synchronize()
    refe = oracle.extend(host(k, used), host(v, used), to_numpy_storage(qe), q_start,
                         np.searchsorted(used, ids).astype(np.int32), lens, d ** -0.5)
    _check(_to64(oute), refe, "bf16", "extend over blocks past 4 GiB")

    # slot write into high blocks (one slot per block, so slots are distinct)
    T = 64
    wblk = rng.permutation(hi)[:T]
    rows = rng.integers(0, B, T)
    kn = torch.randn((T, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
    vn = torch.randn((T, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
    kref, vref = oracle.kv_write(host(k, wblk), host(v, wblk), to_numpy_storage(kn),
                                 to_numpy_storage(vn), (np.arange(T) * B + rows).astype(np.int64))
    pk.pa_kv_write(k, v, kn, vn, torch.from_numpy((wblk * B + rows).astype(np.int64)).to(dev))
    torch.cuda.synchronize()
    assert np.array_equal(host(k, wblk), kref)
    assert np.array_equal(host(v, wblk), vref)

    # block copy across the mark both ways: no destination is a source
    P = 16
    src_hi, dst_hi = np.split(rng.permutation(hi)[:2 * P], 2)
    src_lo, dst_lo = np.split(rng.permutation(lo_n)[:2 * P], 2)
    src = np.concatenate([src_hi, src_lo])
    dst = np.concatenate([dst_lo, dst_hi])
    k_src, v_src = host(k, src), host(v, src)
    pk.pa_block_copy(k, v, torch.from_numpy(np.stack([src, dst], 1).astype(np.int32)).to(dev))
    torch.cuda.synchronize()
    assert np.array_equal(host(k, dst), k_src)
    assert np.array_equal(host(v, dst), v_src)
    del k, v
    torch.cuda.empty_cache()


def test_write_and_decode_replayed_from_a_hip_graph(pk):
    """A decode step's device work -- slot write, then decode with a caller
    workspace -- captured once in a HIP graph (the calls allocate, memset
    and synchronize nothing) and replayed three times.  Between replays the
    program writes new queries, new token rows and new slots eagerly; every
    replay must equal the same two calls run eagerly on a second copy of the
    pools, bit for bit."""
    rng = np.random.default_rng(77)
    lens = (5, 16, 17, 200, 700)
    c = _custom_case(lens, Hq=8, Hkv=2, d=128, nb=300, width=44, seed=78)
    k, v = c.k_pool, c.v_pool
    kr, vr = k.clone(), v.clone()
    T = 8
    kn = torch.empty((T, 2, 128), dtype=torch.bfloat16, device="cuda")
    vn = torch.empty_like(kn)
    slots = torch.empty(T, dtype=torch.int64, device="cuda")
    q = c.q.clone()
    out = torch.empty_like(q)
    S, maxB = len(lens), c.block_tables.shape[1]
    ws = torch.empty(pk.pa_decode_workspace_bytes(k, v, S, 8, maxB), dtype=torch.uint8,
                     device="cuda")

    def fill(i):
        g = torch.Generator().manual_seed(1000 + i)
        q.copy_(torch.randn(q.shape, generator=g).to(torch.bfloat16))
        kn.copy_(torch.randn(kn.shape, generator=g).to(torch.bfloat16))
        vn.copy_(torch.randn(vn.shape, generator=g).to(torch.bfloat16))
        slots.copy_(torch.from_numpy(rng.permutation(300 * 16)[:T].astype(np.int64)))

    def step(kp, vp, o, w):
        pk.pa_kv_write(kp, vp, kn, vn, slots)
        pk.pa_decode(q, kp, vp, c.block_tables, c.context_lens, c.scale, out=o, workspace=w)

    fill(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(k, v, out, ws)            # warm-up before capture (launch set-up done once)
        step(kr, vr, torch.empty_like(out), ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(k, v, out, ws)
    ws_ref = torch.empty_like(ws)
    for i in range(1, 4):
        fill(i)
        torch.cuda.synchronize()
        graph.replay()
        ref = torch.empty_like(out)
        step(kr, vr, ref, ws_ref)
        torch.cuda.synchronize()
        assert torch.equal(k, kr) and torch.equal(v, vr), f"replay {i}: pools differ"
        assert torch.equal(out, ref), f"replay {i}: decode output differs"
        assert torch.isfinite(out.float()).all()


# --- full-size configs: every output ------------------------------------------
FULL = ["llama2_7b_mha", "llama3_8b_gqa", "prefix_sharing", "long_context_128k"]


@pytest.mark.slow
@pytest.mark.parametrize("key", FULL)
def test_decode_full_size_all_outputs(pk, key):
    """The configuration at its full size, in the launch configuration the
    benchmark uses: every (sequence, head) output against the oracle, and a
    second call bit-identical to the first."""
    cfg = CONFIGS[key]
    _log(f"{key}: generating on the GPU")
    c = decode_case(cfg, payload="torch", device="cuda")
    got = _gpu_decode(pk, c, cfg.partition_tokens).clone()
    assert torch.equal(got, _gpu_decode(pk, c, cfg.partition_tokens)), f"{key}: not deterministic"
    S, Hq = cfg.num_seqs, cfg.num_q_heads
    pairs = np.array([[s, h] for s in range(S) for h in range(Hq)], np.int32)
    _log(f"{key}: copying pools to the host for all {len(pairs)} outputs")
    ref = oracle.decode_pairs(*c.oracle_inputs(), c.scale, pairs)
    g64 = _to64(got)
    _check(g64[pairs[:, 0], pairs[:, 1]], ref, cfg.dtype, f"{key} full size, all outputs")
    del c
    torch.cuda.empty_cache()


# --- slot write, block copy, table update: bit-exact --------------------------
@pytest.mark.parametrize("dtype,T,skip", [("bf16", 256, 0.0), ("bf16", 1000, 0.2),
                                          ("f32", 77, 0.1), ("bf16", 1, 0.0)])
def test_kv_write_bit_exact(pk, dtype, T, skip):
    w = kv_write_case(200, 8, 128, 16, T, dtype=dtype, skip_fraction=skip, seed=T)
    kref, vref = oracle.kv_write(w.k_pool, w.v_pool, w.k_new, w.v_new, w.slot_mapping)
    k = from_numpy_storage(w.k_pool, dtype, "cuda")
    v = from_numpy_storage(w.v_pool, dtype, "cuda")
    pk.pa_kv_write(k, v, from_numpy_storage(w.k_new, dtype, "cuda"),
                   from_numpy_storage(w.v_new, dtype, "cuda"),
                   torch.from_numpy(w.slot_mapping).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(to_numpy_storage(k), kref)
    assert np.array_equal(to_numpy_storage(v), vref)


def test_kv_write_odd_head_dim_bit_exact(pk):
    w = kv_write_case(40, 3, 12, 16, 50, dtype="bf16", skip_fraction=0.1, seed=9)
    kref, vref = oracle.kv_write(w.k_pool, w.v_pool, w.k_new, w.v_new, w.slot_mapping)
    k = from_numpy_storage(w.k_pool, "bf16", "cuda")
    v = from_numpy_storage(w.v_pool, "bf16", "cuda")
    pk.pa_kv_write(k, v, from_numpy_storage(w.k_new, "bf16", "cuda"),
                   from_numpy_storage(w.v_new, "bf16", "cuda"),
                   torch.from_numpy(w.slot_mapping).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(to_numpy_storage(k), kref)
    assert np.array_equal(to_numpy_storage(v), vref)


@pytest.mark.parametrize("dtype,P", [("bf16", 192), ("f32", 5), ("bf16", 1)])
def test_block_copy_bit_exact(pk, dtype, P):
    c = block_copy_case(400, 8, 128, 16, P, dtype=dtype, seed=P)
    kref, vref = oracle.block_copy(c.k_pool, c.v_pool, c.pairs)
    k = from_numpy_storage(c.k_pool, dtype, "cuda")
    v = from_numpy_storage(c.v_pool, dtype, "cuda")
    pk.pa_block_copy(k, v, torch.from_numpy(c.pairs).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(to_numpy_storage(k), kref)
    assert np.array_equal(to_numpy_storage(v), vref)


def test_table_update_bit_exact(pk):
    rng = np.random.default_rng(3)
    S, W, B = 20, 12, 16
    tables = rng.integers(0, 500, (S, W)).astype(np.int32)
    T = 40
    seq = rng.integers(0, S, T).astype(np.int32)
    pos = rng.integers(0, W * B, T).astype(np.int32)
    # distinct (seq, entry) so the result is unique
    key = seq.astype(np.int64) * W + pos // B
    _, first = np.unique(key, return_index=True)
    seq, pos = seq[first], pos[first]
    slots = rng.integers(0, 500 * B, len(seq)).astype(np.int64)
    slots[::7] = -1
    expect = tables.copy()
    for s_, p_, sl in zip(seq, pos, slots):
        if sl >= 0:
            expect[s_, p_ // B] = sl // B
    t = torch.from_numpy(tables).cuda()
    pk.pa_table_update(t, B, torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(),
                       torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(t.cpu().numpy(), expect)


def test_kv_append_bit_exact(pk):
    """Append = table update + slot write in one launch: the pools match the
    oracle's slot write and the table the update rule, bit for bit."""
    rng = np.random.default_rng(12)
    nb, Hkv, d, B, S, W = 300, 8, 128, 16, 24, 20
    w = kv_write_case(nb, Hkv, d, B, 0, dtype="bf16", seed=13)
    # one token per sequence at a random position, into distinct random slots
    T = S
    seq = np.arange(S, dtype=np.int32)
    pos = rng.integers(0, W * B, T).astype(np.int32)
    slots = rng.permutation(nb * B)[:T].astype(np.int64)
    slots[::5] = -1
    k_new = rng.standard_normal((T, Hkv, d), dtype=np.float32)
    v_new = rng.standard_normal((T, Hkv, d), dtype=np.float32)
    kn = torch.from_numpy(k_new).to(torch.bfloat16)
    vn = torch.from_numpy(v_new).to(torch.bfloat16)
    kref, vref = oracle.kv_write(w.k_pool, w.v_pool, to_numpy_storage(kn), to_numpy_storage(vn),
                                 slots)
    tables = rng.integers(0, nb, (S, W)).astype(np.int32)
    expect = tables.copy()
    for s_, p_, sl in zip(seq, pos, slots):
        if sl >= 0:
            expect[s_, p_ // B] = sl // B
    k = from_numpy_storage(w.k_pool, "bf16", "cuda")
    v = from_numpy_storage(w.v_pool, "bf16", "cuda")
    t = torch.from_numpy(tables).cuda()
    pk.pa_kv_append(k, v, kn.cuda(), vn.cuda(), torch.from_numpy(slots).cuda(), t,
                    torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(to_numpy_storage(k), kref)
    assert np.array_equal(to_numpy_storage(v), vref)
    assert np.array_equal(t.cpu().numpy(), expect)


# --- the whole path: block manager -> copy -> write -> decode -----------------
def _run_path_both(pk, prompts, samples, shared, private_lo, private_hi, Hq, Hkv, d, seed,
                   decode_steps=3, kv="bf16"):
    """Each side runs its own block manager and kernels from the same seeded
    token K/V; tables/slots/pairs must match exactly, pools bit for bit, and
    attention within tolerance.  kv="fp8": 8-bit pools (tokens stay bf16 and
    are quantised by each side's slot write)."""
    B = 16
    rng = np.random.default_rng(seed)
    privs = rng.integers(private_lo, private_hi, prompts * samples, endpoint=True)
    nb = prompts * (shared // B + 2) + int(((privs + decode_steps) // B + 2).sum())
    bm_seed = seed * 7 + 1
    cbm = pk.BlockManager(nb, B, bm_seed)
    mbm = BlockManagerModel(nb, B, bm_seed)
    dt = torch.bfloat16
    if kv == "fp8":
        rk, rv = fp8_region_bytes(B, d)
        k_host = np.zeros((nb, Hkv, rk), np.uint8)
        v_host = np.zeros((nb, Hkv, rv), np.uint8)
        fp8_poison(k_host, v_host, np.ones((nb, B), bool), B, d)
        k_dev = torch.from_numpy(k_host).cuda()
        v_dev = torch.from_numpy(v_host).cuda()
    else:
        k_dev = torch.full((nb, Hkv, B, d), 64.0, dtype=dt, device="cuda")
        v_dev = torch.full((nb, Hkv, d, B), POISON_V, dtype=dt, device="cuda")
        k_host = to_numpy_storage(k_dev)
        v_host = to_numpy_storage(v_dev)

    def tokens(n):
        kn = torch.from_numpy(rng.standard_normal((n, Hkv, d), dtype=np.float32)).to(dt)
        vn = torch.from_numpy(rng.standard_normal((n, Hkv, d), dtype=np.float32)).to(dt)
        return kn, vn

    def both_append(seqs, ns):
        nonlocal k_host, v_host
        st, slots, sq, pos, pairs = cbm.append_batch(seqs, ns)
        assert st == pk.PA_OK
        m_slots, m_pairs = [], []
        for s, n in zip(seqs, ns):
            r = mbm.append(s, n)
            m_slots += r[1]
            m_pairs += r[2]
        assert slots.tolist() == m_slots
        assert [tuple(x) for x in pairs.tolist()] == m_pairs
        kn, vn = tokens(len(slots))
        if len(pairs):
            pk.pa_block_copy(k_dev, v_dev, torch.from_numpy(pairs).cuda())
            k_host, v_host = oracle.block_copy(k_host, v_host, np.array(m_pairs, np.int32))
        pk.pa_kv_write(k_dev, v_dev, kn.cuda(), vn.cuda(), torch.from_numpy(slots).cuda())
        k_host, v_host = oracle.kv_write(k_host, v_host, to_numpy_storage(kn),
                                         to_numpy_storage(vn), np.array(m_slots, np.int64))
        return slots, sq, pos, len(pairs)

    seqs = []
    n_cow = 0
    for p in range(prompts):
        root = cbm.add_seq()
        assert mbm.add_seq() == root
        both_append([root], [shared])
        kids = [root]
        for _ in range(samples - 1):
            st, kid = cbm.fork(root)
            assert mbm.fork(root) == (st, kid)
            kids.append(kid)
        _, _, _, nc = both_append(kids, [int(privs[p * samples + i]) for i in range(samples)])
        n_cow += nc
        seqs += kids
    width = int(np.max([mbm.seqs[s].n_tokens for s in seqs]) + decode_steps) // B + 2
    tables_dev = None
    for step in range(decode_steps):
        slots, sq, pos, _ = both_append(seqs, [1] * len(seqs))
        if tables_dev is None:
            tables, lens = cbm.export(seqs, width, pad_block=0)
            tables_dev = torch.from_numpy(tables).cuda()
        else:
            # device mirror follows growth through the table update kernel
            idx = np.searchsorted(np.array(seqs), sq)
            pk.pa_table_update(tables_dev, B, torch.from_numpy(idx.astype(np.int32)).cuda(),
                               torch.from_numpy(pos).cuda(), torch.from_numpy(slots).cuda())
            tables, lens = cbm.export(seqs, width, pad_block=0)
        torch.cuda.synchronize()
        assert np.array_equal(tables_dev.cpu().numpy(), tables)
        m_tab = np.zeros_like(tables)
        for i, s in enumerate(seqs):
            m_tab[i, :len(mbm.seqs[s].table)] = mbm.seqs[s].table
        assert np.array_equal(m_tab, tables)
        q = torch.from_numpy(rng.standard_normal((len(seqs), Hq, d), dtype=np.float32)).to(dt)
        out = pk.pa_decode(q.cuda(), k_dev, v_dev, tables_dev, torch.from_numpy(lens).cuda(),
                           d ** -0.5)
        torch.cuda.synchronize()
        assert np.array_equal(to_numpy_storage(k_dev), k_host)
        assert np.array_equal(to_numpy_storage(v_dev), v_host)
        ref = oracle.decode(k_host, v_host, to_numpy_storage(q), tables, lens, d ** -0.5)
        _check(_to64(out), ref, "bf16", f"path step {step}")
    return n_cow


def test_full_path_prefix_sharing_with_copy_on_write(pk):
    n_cow = _run_path_both(pk, prompts=4, samples=4, shared=104, private_lo=1, private_hi=40,
                           Hq=32, Hkv=8, d=128, seed=11)
    assert n_cow == 4 * 3


def test_full_path_full_shared_tail_no_copy(pk):
    n_cow = _run_path_both(pk, prompts=3, samples=4, shared=96, private_lo=1, private_hi=30,
                           Hq=32, Hkv=8, d=128, seed=12)
    assert n_cow == 0


def test_full_path_mha(pk):
    _run_path_both(pk, prompts=6, samples=1, shared=200, private_lo=1, private_hi=300, Hq=8,
                   Hkv=8, d=128, seed=13)


def test_full_path_fp8_cache_with_copy_on_write(pk):
    n_cow = _run_path_both(pk, prompts=4, samples=4, shared=104, private_lo=1, private_hi=40,
                           Hq=32, Hkv=8, d=128, seed=14, kv="fp8")
    assert n_cow == 4 * 3


# --- error paths ---------------------------------------------------------------
def test_debug_validation_rejects_bad_device_indices(pk, monkeypatch):
    cfg = SMALL["llama3_8b_gqa"]
    c = decode_case(cfg, payload="numpy", device="cuda")
    monkeypatch.setenv("PA_DEBUG", "1")
    bad = c.context_lens.clone()
    bad[0] = 0
    with pytest.raises(pk.PagedKVError) as e:
        pk.pa_decode(c.q, c.k_pool, c.v_pool, c.block_tables, bad, c.scale)
    assert e.value.status == pk.PA_EINVAL
    badt = c.block_tables.clone()
    badt[0, 0] = c.num_blocks
    with pytest.raises(pk.PagedKVError):
        pk.pa_decode(c.q, c.k_pool, c.v_pool, badt, c.context_lens, c.scale)
    dup = torch.tensor([3, 3], dtype=torch.int64, device="cuda")
    kn = torch.zeros(2, cfg.num_kv_heads, cfg.head_dim, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(pk.PagedKVError):
        pk.pa_kv_write(c.k_pool, c.v_pool, kn, kn, dup)
    pairs = torch.tensor([[1, 2], [2, 3]], dtype=torch.int32, device="cuda")
    with pytest.raises(pk.PagedKVError):
        pk.pa_block_copy(c.k_pool, c.v_pool, pairs)
    # valid inputs still pass with validation on
    pk.pa_decode(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens, c.scale)
    torch.cuda.synchronize()
