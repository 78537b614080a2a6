"""GPU parity of multi-token paged attention (extend / chunked prefill with
a causal mask): the HIP path through the C-ABI against the CPU oracle on the
same seeded inputs; max |GPU - oracle| <= 2e-2 on every output (bf16)."""
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads.gen import f32_to_bf16_bits, to_numpy_storage

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def pk():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import paged_kv_cache_335_amd as pk
    return pk


def _case(rng, lens, ns, Hq, Hkv, d, nb=None, B=16):
    """Random bf16 pools and tables; unused slots hold NaN-free random data."""
    S = len(lens)
    width = max(1, max(-(-L // B) for L in lens))
    nb = nb or max(64, width * S + 8)
    k = f32_to_bf16_bits(rng.standard_normal((nb, Hkv, B, d), dtype=np.float32))
    v = f32_to_bf16_bits(rng.standard_normal((nb, Hkv, d, B), dtype=np.float32))
    tables = np.stack([rng.permutation(nb)[:width] for _ in range(S)]).astype(np.int32)
    q_start = np.concatenate([[0], np.cumsum(ns)]).astype(np.int32)
    q = f32_to_bf16_bits(rng.standard_normal((int(q_start[-1]), Hq, d), dtype=np.float32))
    return k, v, q, q_start, tables, np.asarray(lens, np.int32)


def _dev(a, bf16=False):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if bf16:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.cuda()


def _run(pk, k, v, q, qs, tables, lens, scale, workspace=None):
    out = pk.pa_extend(_dev(q, True), _dev(k, True), _dev(v, True), _dev(qs), _dev(tables),
                       _dev(lens), scale, workspace=workspace)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("G,d", [(1, 128), (2, 64), (4, 128), (8, 128), (16, 64), (3, 128)])
def test_extend_matches_oracle(pk, G, d):
    rng = np.random.default_rng(300 + G + d)
    # prefill from empty (n = L), short extends, single queries, multi-tile chunks
    lens = [37, 1, 130, 64, 300, 17, 256, 5]
    ns = [37, 1, 20, 1, 77, 16, 256, 0]
    Hkv = 2
    k, v, q, qs, tables, lens = _case(rng, lens, ns, G * Hkv, Hkv, d)
    ref = oracle.extend(k, v, q, qs, tables, lens, d ** -0.5)
    got = _run(pk, k, v, q, qs, tables, lens, d ** -0.5)
    err = np.abs(got - ref)
    _log(f"G={G} d={d}: max|err| {err.max():.3e}")
    assert np.isfinite(got).all() and err.max() <= 2e-2


@pytest.mark.parametrize("scale", [-0.1, 0.0])
def test_extend_non_positive_scale(pk, scale):
    """A positive scale takes the kernel's fused scale-and-subtract form; a
    negative or zero scale takes the plain one (zero: uniform weights over
    each row's visible tokens)."""
    rng = np.random.default_rng(91)
    lens, ns = [37, 300, 64, 17], [37, 77, 1, 16]
    k, v, q, qs, tables, lens = _case(rng, lens, ns, 8, 2, 128)
    ref = oracle.extend(k, v, q, qs, tables, lens, scale)
    got = _run(pk, k, v, q, qs, tables, lens, scale)
    err = np.abs(got - ref)
    _log(f"scale {scale}: max|err| {err.max():.3e}")
    assert np.isfinite(got).all() and err.max() <= 2e-2


@pytest.mark.parametrize("d", [128, 64])
def test_extend_contexts_longer_than_one_table_window(pk, d):
    """Contexts of 1250 and 1025 blocks: the kernel stages the block table
    1024 entries at a time, so these rows read through a second window (and
    the second one holds a single block).  Every output against the oracle."""
    rng = np.random.default_rng(77 + d)
    lens, ns = [20000, 16400, 300], [70, 5, 33]
    k, v, q, qs, tables, lens = _case(rng, lens, ns, 8, 2, d, nb=1300)
    ref = oracle.extend(k, v, q, qs, tables, lens, d ** -0.5)
    got = _run(pk, k, v, q, qs, tables, lens, d ** -0.5)
    err = np.abs(got - ref)
    _log(f"long contexts d={d}: max|err| {err.max():.3e}")
    assert np.isfinite(got).all() and err.max() <= 2e-2


@pytest.mark.parametrize("G,d", [(4, 128), (8, 64), (1, 128)])
def test_extend_context_split_long_prefixes(pk, G, d):
    """Few sequences with long cached prefixes: too few units to fill the
    chip, so the library cuts each context into chunks (partials + combine).
    The split result and the unsplit one (a workspace too small to hold the
    partials) both match the oracle; unused slots of the last blocks hold
    NaN, which no chunk may let through."""
    rng = np.random.default_rng(340 + G + d)
    Hkv = 2
    lens, ns = [30000, 9001, 1500], [40, 7, 1]
    width = -(-max(lens) // 16)
    k, v, q, qs, tables, lens = _case(rng, lens, ns, G * Hkv, Hkv, d, nb=2 * width + 200)
    # tables of different sequences may share blocks: NaN only where no
    # sequence reads
    used = np.zeros((k.shape[0], 16), bool)
    for s, L in enumerate(lens):
        for t0 in range(0, L, 16):
            used[tables[s, t0 // 16], :min(16, L - t0)] = True
    nan = f32_to_bf16_bits(np.array([np.nan], np.float32))[0]
    for s, L in enumerate(lens):
        b = tables[s, (L - 1) // 16]
        for r in np.flatnonzero(~used[b]):
            k[b, :, r, :] = nan
            v[b, :, :, r] = nan
    ws = pk.pa_extend_workspace_bytes(_dev(k, True), _dev(v, True), int(qs[-1]), len(lens),
                                      G * Hkv, tables.shape[1])
    assert ws > 0, "this batch should take the split path"
    ref = oracle.extend(k, v, q, qs, tables, lens, d ** -0.5)
    split = _run(pk, k, v, q, qs, tables, lens, d ** -0.5)
    whole = _run(pk, k, v, q, qs, tables, lens, d ** -0.5,
                 workspace=torch.empty(1, dtype=torch.uint8, device="cuda"))
    for name, got in (("split", split), ("whole", whole)):
        err = np.abs(got - ref)
        _log(f"G={G} d={d} {name}: max|err| {err.max():.3e}")
        assert np.isfinite(got).all() and err.max() <= 2e-2


def test_extend_many_sequences_and_determinism(pk):
    rng = np.random.default_rng(310)
    S = 200
    lens = rng.integers(1, 400, S)
    ns = np.minimum(lens, rng.integers(0, 40, S))
    k, v, q, qs, tables, lens = _case(rng, lens.tolist(), ns.tolist(), 32, 8, 128, nb=4000)
    ref = oracle.extend(k, v, q, qs, tables, lens, 128 ** -0.5)
    a = _run(pk, k, v, q, qs, tables, lens, 128 ** -0.5)
    b = _run(pk, k, v, q, qs, tables, lens, 128 ** -0.5)
    assert np.array_equal(a, b)
    assert np.abs(a - ref).max() <= 2e-2


def test_extend_work_order_mixed_lengths(pk):
    """Units go out longest sequence first (a sort of up to 1024 sequences
    in LDS) in a snake over the grid: every unit exactly once whatever the
    order.  A batch of widely mixed lengths with some query-less sequences,
    then one past the sort's limit (sequence order), both against the
    oracle."""
    rng = np.random.default_rng(350)
    for S, Lmax in ((300, 3000), (1100, 80)):
        lens = np.maximum(1, (rng.lognormal(0, 1.2, S) * Lmax / 8).astype(int))
        lens = np.minimum(lens, Lmax)
        ns = np.minimum(lens, rng.integers(0, 24, S))
        ns[rng.random(S) < 0.2] = 0
        k, v, q, qs, tables, lens = _case(rng, lens.tolist(), ns.tolist(), 8, 2, 128,
                                          nb=max(4000, int(lens.sum()) // 16 + 64))
        ref = oracle.extend(k, v, q, qs, tables, lens, 128 ** -0.5)
        got = _run(pk, k, v, q, qs, tables, lens, 128 ** -0.5)
        err = np.abs(got - ref)
        _log(f"S={S}: max|err| {err.max():.3e}")
        assert np.isfinite(got).all() and err.max() <= 2e-2


def test_extend_nan_in_unused_slots_never_reaches_output(pk):
    """Slots past each context (the tail of the last block, unused blocks)
    hold NaN: masked tokens contribute nothing."""
    rng = np.random.default_rng(320)
    lens, ns = [21, 50], [21, 9]
    k, v, q, qs, tables, lens = _case(rng, lens, ns, 8, 2, 128, nb=20)
    ref = oracle.extend(k, v, q, qs, tables, lens, 0.1)
    kf = k.copy()
    vf = v.copy()
    used = np.zeros((20, 16), bool)
    for s, L in enumerate(lens):
        for t in range(L):
            used[tables[s, t // 16], t % 16] = True
    nan = f32_to_bf16_bits(np.array([np.nan], np.float32))[0]
    for b in range(20):
        for r in range(16):
            if not used[b, r]:
                kf[b, :, r, :] = nan
                vf[b, :, :, r] = nan
    got = _run(pk, kf, vf, q, qs, tables, lens, 0.1)
    assert np.isfinite(got).all() and np.abs(got - ref).max() <= 2e-2


def test_chunked_prefill_through_the_runtime(pk):
    """Three sequences prefilled in chunks of 48 tokens through the runtime
    (block manager -> slot write -> extend); each chunk's output against the
    oracle over the oracle's own copy of the cache."""
    from paged_kv_cache_335_amd.runtime import PagedKVCache
    rng = np.random.default_rng(330)
    Hq, Hkv, d, B = 16, 4, 128, 16
    cache = PagedKVCache(200, Hkv, d, 8, 64, block_size=B, shuffle_seed=3)
    seqs = [cache.add_sequence() for _ in range(3)]
    total = [150, 97, 48]
    k_host = to_numpy_storage(torch.zeros_like(cache.k_pool))
    v_host = to_numpy_storage(torch.zeros_like(cache.v_pool))
    cache.k_pool.zero_()
    cache.v_pool.zero_()
    done = [0, 0, 0]
    while any(dn < t for dn, t in zip(done, total)):
        ns = [min(48, t - dn) for dn, t in zip(done, total)]
        T = sum(ns)
        kn = f32_to_bf16_bits(rng.standard_normal((T, Hkv, d), dtype=np.float32))
        vn = f32_to_bf16_bits(rng.standard_normal((T, Hkv, d), dtype=np.float32))
        q = f32_to_bf16_bits(rng.standard_normal((T, Hq, d), dtype=np.float32))
        out = cache.extend(seqs, ns, _dev(q, True), _dev(kn, True), _dev(vn, True))
        torch.cuda.synchronize()
        tables, lens = cache.bm.export(np.array(seqs, np.int32), 64, pad_block=0)
        slots = []
        for i, s in enumerate(seqs):
            for j in range(ns[i]):
                pos = done[i] + j
                slots.append(int(tables[i, pos // B]) * B + pos % B)
        k_host, v_host = oracle.kv_write(k_host, v_host, kn, vn, np.array(slots, np.int64))
        assert np.array_equal(to_numpy_storage(cache.k_pool), k_host)
        qs = np.concatenate([[0], np.cumsum(ns)]).astype(np.int32)
        ref = oracle.extend(k_host, v_host, q, qs, tables, lens, d ** -0.5)
        err = np.abs(out.float().cpu().numpy() - ref).max()
        _log(f"chunk {done}: max|err| {err:.3e}")
        assert err <= 2e-2
        done = [dn + n for dn, n in zip(done, ns)]
