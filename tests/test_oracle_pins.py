"""Pins for the numeric oracle: each test fixes the oracle to something other
than itself (a worked example from the pages, a closed form, an invariant the
pages state, or a textbook library routine on a special case), chosen so that
a plausible slip in the oracle (wrong table index, wrong head mapping, a
transposed V, a dropped scale, no max subtraction, reading masked slots)
fails at least one of them.  CPU only."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from workloads import bf16_bits_to_f32, f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _pools(nb, nkv, B, d, rng, dtype="f32"):
    k = rng.standard_normal((nb, nkv, B, d)).astype(np.float32)
    v = rng.standard_normal((nb, nkv, d, B)).astype(np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    return k, v


def _f(x):
    return bf16_bits_to_f32(x) if x.dtype == np.uint16 else x


# --- worked example: the page table keeps pages in order -------------------
def test_gather_follows_table_keep_pages_in_order():
    g = json.load(open(os.path.join(GOLDEN, "keep_pages_in_order.json")))
    nb, B = g["num_blocks"], g["block_size"]
    k = np.zeros((nb, 1, B, 2), np.float32)
    v = np.zeros((nb, 1, 2, B), np.float32)
    for blk, text in g["blocks"].items():
        assert len(text) == B
        for r, ch in enumerate(text):
            k[int(blk), 0, r] = [ord(ch), r]
            v[int(blk), 0, :, r] = [ord(ch), -ord(ch)]
    table = np.array(g["table"], np.int32)
    L = len(table) * B
    Kc, Vc = oracle.gather(k, v, table, 0, L)
    text_k = "".join(chr(int(c)) for c in Kc[:, 0])
    text_v = "".join(chr(int(c)) for c in Vc[:, 0])
    assert text_k == g["expected_text"]
    assert text_v == g["expected_text"]
    assert np.array_equal(Vc[:, 1], -Vc[:, 0])
    assert np.array_equal(Kc[:, 1], np.tile(np.arange(B), len(table)))


# --- closed forms -----------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_token_returns_its_value_row(dtype):
    """L = 1: softmax of one score is 1, so out = V_0 exactly."""
    rng = np.random.default_rng(10)
    nb, nkv, B, d, Hq = 6, 2, 4, 8, 4
    k, v = _pools(nb, nkv, B, d, rng, dtype)
    q = rng.standard_normal((3, Hq, d)).astype(np.float32)
    q = f32_to_bf16_bits(q) if dtype == "bf16" else q
    tables = np.array([[5, 0], [2, 1], [4, 3]], np.int32)
    lens = np.array([1, 1, 1], np.int32)
    out = oracle.decode(k, v, q, tables, lens, 0.3)
    vf = _f(v)
    G = Hq // nkv
    for s in range(3):
        for h in range(Hq):
            expect = vf[tables[s, 0], h // G, :, 0].astype(np.float64)
            assert np.array_equal(out[s, h], expect)


def test_equal_keys_give_mean_of_values():
    rng = np.random.default_rng(11)
    nb, B, d, L = 5, 4, 16, 13
    k, v = _pools(nb, 1, B, d, rng)
    row = rng.standard_normal(d).astype(np.float32)
    k[:] = row
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    table = np.array([[3, 0, 4, 1]], np.int32)
    out = oracle.decode(k, v, q, table, np.array([L], np.int32), 0.7)
    Kc, Vc = oracle.gather(k, v, table[0], 0, L)
    assert np.allclose(out[0, 0], Vc.mean(axis=0), rtol=0, atol=1e-13)


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(12)
    nb, B, d, L = 4, 4, 8, 10
    k, v = _pools(nb, 1, B, d, rng)
    q = np.zeros((1, 1, d), np.float32)
    table = np.array([[2, 0, 3]], np.int32)
    out = oracle.decode(k, v, q, table, np.array([L], np.int32), 1.0)
    # mean written out per element from the layout: token t lives in block
    # table[t // B] at slot t % B, V stored dim-major
    expect = np.zeros(d)
    for t in range(L):
        expect += v[table[0, t // B], 0, :, t % B]
    assert np.allclose(out[0, 0], expect / L, rtol=0, atol=1e-13)


def test_two_tokens_logistic_closed_form():
    """L = 2: out = sigmoid(D) V0 + sigmoid(-D) V1, D = scale q.(k0 - k1)."""
    d, B, scale = 4, 2, 0.37
    k = np.zeros((1, 1, B, d), np.float32)
    v = np.zeros((1, 1, d, B), np.float32)
    k[0, 0, 0] = [1.0, 2.0, -1.0, 0.5]
    k[0, 0, 1] = [0.0, -1.0, 3.0, 1.0]
    v[0, 0, :, 0] = [1.0, 0.0, 2.0, -3.0]
    v[0, 0, :, 1] = [-1.0, 4.0, 0.0, 1.0]
    q = np.array([[[0.5, -1.0, 2.0, 1.5]]], np.float32)
    out = oracle.decode(k, v, q, np.array([[0]], np.int32), np.array([2], np.int32), scale)
    D = scale * float(q[0, 0] @ (k[0, 0, 0] - k[0, 0, 1]))
    sig = 1.0 / (1.0 + math.exp(-D))
    v0, v1 = v[0, 0, :, 0].astype(np.float64), v[0, 0, :, 1].astype(np.float64)
    expect = sig * v0 + (1 - sig) * v1
    assert np.allclose(out[0, 0], expect, rtol=0, atol=1e-14)
    # the sign of D matters: swapping the keys must change the answer
    assert not np.allclose(out[0, 0], (1 - sig) * v0 + sig * v1)


def test_dominant_score_picks_its_row_without_overflow():
    """Scores of order 1e4: exp without max subtraction overflows; with it,
    all weight lands on the arg-max token."""
    d, B, L = 4, 4, 7
    k = np.zeros((2, 1, B, d), np.float32)
    v = np.arange(2 * d * B, dtype=np.float32).reshape(2, 1, d, B)
    k[1, 0, 2] = [100.0, 0, 0, 0]          # logical token 6 (block 1 at index 1, slot 2)
    k[0, 0, :, 0] = 10.0
    k[1, 0, 0:2, 0] = 10.0
    q = np.array([[[100.0, 0, 0, 0]]], np.float32)
    table = np.array([[0, 1]], np.int32)
    out = oracle.decode(k, v, q, table, np.array([L], np.int32), 1.0)
    assert np.all(np.isfinite(out))
    assert np.array_equal(out[0, 0], v[1, 0, :, 2].astype(np.float64))


def test_gqa_head_mapping_uses_consecutive_groups():
    """With 8 query heads over 2 KV heads, heads 0-3 read KV head 0 and heads
    4-7 read KV head 1 (several query heads share one K/V set)."""
    rng = np.random.default_rng(13)
    nb, nkv, B, d, Hq, L = 3, 2, 4, 8, 8, 9
    k, v = _pools(nb, nkv, B, d, rng)
    v[:, 0] = 1.0
    v[:, 1] = -1.0
    q = rng.standard_normal((1, Hq, d)).astype(np.float32)
    out = oracle.decode(k, v, q, np.array([[2, 0, 1]], np.int32), np.array([L], np.int32),
                        0.5)
    assert np.allclose(out[0, :4], 1.0, atol=1e-14)
    assert np.allclose(out[0, 4:], -1.0, atol=1e-14)


def test_matches_textbook_softmax_library_routine():
    """Random case against scipy's softmax and a numpy matrix product on the
    contiguous copy read straight from the layout."""
    from scipy.special import softmax
    rng = np.random.default_rng(14)
    nb, nkv, B, d, Hq = 12, 2, 4, 16, 6
    k, v = _pools(nb, nkv, B, d, rng, "bf16")
    q = f32_to_bf16_bits(rng.standard_normal((2, Hq, d)).astype(np.float32))
    tables = np.array([[7, 3, 11, 0], [1, 9, 2, 5]], np.int32)
    lens = np.array([15, 6], np.int32)
    scale = 1 / math.sqrt(d)
    out = oracle.decode(k, v, q, tables, lens, scale)
    kf, vf, qf = (bf16_bits_to_f32(x).astype(np.float64) for x in (k, v, q))
    G = Hq // nkv
    for s in range(2):
        L = lens[s]
        pos = np.arange(L)
        blk, slot = tables[s, pos // B], pos % B
        for h in range(Hq):
            K = kf[blk, h // G, slot, :]          # [L][d]
            V = vf[blk, h // G, :, slot]          # [L][d]
            p = softmax(scale * (K @ qf[s, h]))
            assert np.allclose(out[s, h], p @ V, rtol=0, atol=1e-12)


# --- invariants the pages state ---------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_paging_does_not_change_outputs_dense_equals_paged(dtype):
    """The attention equation is unchanged by paging: the same logical data
    in a contiguous unpaged layout gives the identical result, bit for bit."""
    rng = np.random.default_rng(15)
    nb, nkv, B, d, Hq, S = 20, 2, 4, 8, 4, 3
    k, v = _pools(nb, nkv, B, d, rng, dtype)
    qf = rng.standard_normal((S, Hq, d)).astype(np.float32)
    q = f32_to_bf16_bits(qf) if dtype == "bf16" else qf
    perm = rng.permutation(nb).astype(np.int32)
    tables = perm[:S * 5].reshape(S, 5)
    lens = np.array([17, 4, 20], np.int32)
    maxL = 20
    kd = np.zeros((S, nkv, maxL, d), k.dtype)
    vd = np.zeros((S, nkv, maxL, d), v.dtype)
    for s in range(S):
        for t in range(lens[s]):
            b, r = tables[s, t // B], t % B
            kd[s, :, t, :] = k[b, :, r, :]
            vd[s, :, t, :] = v[b, :, :, r]
    paged = oracle.decode(k, v, q, tables, lens, 0.25)
    dense = oracle.decode_dense(kd, vd, q, lens, 0.25)
    assert np.array_equal(paged, dense)


def test_physical_placement_is_invisible_bit_exact():
    """Moving blocks to other physical ids (and updating the table) leaves
    every output bit unchanged: only logical positions matter."""
    rng = np.random.default_rng(16)
    nb, nkv, B, d, Hq, S = 16, 1, 4, 8, 2, 2
    k, v = _pools(nb, nkv, B, d, rng, "bf16")
    q = f32_to_bf16_bits(rng.standard_normal((S, Hq, d)).astype(np.float32))
    tables = np.array([[0, 1, 2, 3], [4, 5, 6, 7]], np.int32)
    lens = np.array([14, 16], np.int32)
    out1 = oracle.decode(k, v, q, tables, lens, 0.3)
    move = rng.permutation(nb)
    k2 = np.empty_like(k)
    v2 = np.empty_like(v)
    k2[move] = k
    v2[move] = v
    out2 = oracle.decode(k2, v2, q, move[tables].astype(np.int32), lens, 0.3)
    assert np.array_equal(out1, out2)


def test_masked_slots_do_not_matter():
    """Slots past the context (tail of the last block) and padded table
    entries never contribute: changing them changes no output bit."""
    rng = np.random.default_rng(17)
    nb, nkv, B, d, Hq = 6, 1, 4, 8, 1
    k, v = _pools(nb, nkv, B, d, rng)
    q = rng.standard_normal((1, Hq, d)).astype(np.float32)
    tables = np.array([[4, 1, 5, 0]], np.int32)       # entries 2,3 are padding for L=6
    lens = np.array([6], np.int32)
    out1 = oracle.decode(k, v, q, tables, lens, 0.4)
    k[1, :, 2:, :] = 64.0
    v[1, :, :, 2:] = 1024.0
    k[[5, 0]] = 1e30
    v[[5, 0]] = np.nan
    out2 = oracle.decode(k, v, q, tables, lens, 0.4)
    assert np.array_equal(out1, out2)


@pytest.mark.parametrize("P", [4, 8, 12, 64])
def test_split_context_identity(P):
    """Partition the context, keep (max, sum-exp, unnormalised output) per
    partition, then combine: equal to the unsplit result within 1e-12."""
    rng = np.random.default_rng(18)
    nb, nkv, B, d, Hq, S = 40, 2, 4, 16, 4, 3
    k, v = _pools(nb, nkv, B, d, rng, "bf16")
    q = f32_to_bf16_bits(rng.standard_normal((S, Hq, d)).astype(np.float32) * 3)
    tables = rng.permutation(nb)[:S * 12].reshape(S, 12).astype(np.int32)
    lens = np.array([45, 1, 33], np.int32)
    whole = oracle.decode(k, v, q, tables, lens, 0.25)
    split = oracle.decode_split(k, v, q, tables, lens, 0.25, P)
    assert np.allclose(whole, split, rtol=0, atol=1e-12)


def test_pairs_entry_matches_full_decode():
    rng = np.random.default_rng(19)
    nb, nkv, B, d, Hq, S = 10, 2, 4, 8, 4, 2
    k, v = _pools(nb, nkv, B, d, rng)
    q = rng.standard_normal((S, Hq, d)).astype(np.float32)
    tables = rng.permutation(nb)[:S * 5].reshape(S, 5).astype(np.int32)
    lens = np.array([19, 7], np.int32)
    full = oracle.decode(k, v, q, tables, lens, 0.5)
    pairs = np.array([[1, 3], [0, 0], [1, 1]], np.int32)
    part = oracle.decode_pairs(k, v, q, tables, lens, 0.5, pairs)
    for i, (s, h) in enumerate(pairs):
        assert np.array_equal(part[i], full[s, h])


def test_rejects_out_of_range_block_and_length():
    rng = np.random.default_rng(20)
    k, v = _pools(4, 1, 4, 8, rng)
    q = rng.standard_normal((1, 1, 8)).astype(np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.decode(k, v, q, np.array([[9, 0]], np.int32), np.array([5], np.int32), 1.0)
    with pytest.raises(oracle.OracleError):
        oracle.decode(k, v, q, np.array([[1, 0]], np.int32), np.array([9], np.int32), 1.0)
    with pytest.raises(oracle.OracleError):
        oracle.decode(k, v, q, np.array([[1, 0]], np.int32), np.array([0], np.int32), 1.0)


# --- slot write and block copy ---------------------------------------------
def test_kv_write_layout_by_hand():
    """One token into slot 3 of a 2-block pool with B = 2, d = 2: block 1,
    offset 1.  K is token-major, V dim-major; every other byte stays."""
    k = np.zeros((2, 1, 2, 2), np.float32)
    v = np.zeros((2, 1, 2, 2), np.float32)
    kn = np.array([[[1.0, 2.0]]], np.float32)
    vn = np.array([[[3.0, 4.0]]], np.float32)
    k2, v2 = oracle.kv_write(k, v, kn, vn, np.array([3], np.int64))
    assert k2.ravel().tolist() == [0, 0, 0, 0, 0, 0, 1, 2]
    assert v2.ravel().tolist() == [0, 0, 0, 0, 0, 3, 0, 4]


def test_kv_write_round_trips_through_gather_and_skips_negative_slots():
    rng = np.random.default_rng(21)
    nb, nkv, B, d, T = 8, 2, 4, 8, 6
    k, v = _pools(nb, nkv, B, d, rng, "bf16")
    kn = f32_to_bf16_bits(rng.standard_normal((T, nkv, d)).astype(np.float32))
    vn = f32_to_bf16_bits(rng.standard_normal((T, nkv, d)).astype(np.float32))
    # a sequence whose table is [5, 2]: positions 0..5 -> slots
    table = np.array([5, 2], np.int32)
    slots = np.array([20, 21, 22, 23, 8, 9], np.int64)
    slots_skip = slots.copy()
    slots_skip[4] = -1
    k2, v2 = oracle.kv_write(k, v, kn, vn, slots_skip)
    for g in range(nkv):
        Kc, Vc = oracle.gather(k2, v2, table, g, 6)
        for t in range(6):
            if t == 4:
                # skipped: old content of block 2 slot 0
                assert np.array_equal(Kc[t], bf16_bits_to_f32(k[2, g, 0]))
                continue
            assert np.array_equal(Kc[t], bf16_bits_to_f32(kn[t, g]))
            assert np.array_equal(Vc[t], bf16_bits_to_f32(vn[t, g]))
    # everything not written is unchanged
    touched = np.zeros((nb, B), bool)
    for s in slots_skip[slots_skip >= 0]:
        touched[s // B, s % B] = True
    mask_k = np.broadcast_to(touched[:, None, :, None], k.shape)
    mask_v = np.broadcast_to(touched[:, None, None, :], v.shape)
    assert np.array_equal(k2[~mask_k], k[~mask_k])
    assert np.array_equal(v2[~mask_v], v[~mask_v])


def test_block_copy_gives_sharers_identical_prefix():
    """Copy-on-write: after the copy, a table pointing at the private copy
    reads exactly what the shared block held, and no other block changes."""
    rng = np.random.default_rng(22)
    nb, nkv, B, d = 6, 2, 4, 8
    k, v = _pools(nb, nkv, B, d, rng, "bf16")
    k2, v2 = oracle.block_copy(k, v, np.array([[3, 5], [3, 0]], np.int32))
    for dst in (5, 0):
        for g in range(nkv):
            a = oracle.gather(k2, v2, np.array([1, 3], np.int32), g, 7)
            b = oracle.gather(k2, v2, np.array([1, dst], np.int32), g, 7)
            assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    for blk in (1, 2, 3, 4):
        assert np.array_equal(k2[blk], k[blk]) and np.array_equal(v2[blk], v[blk])


# --- block swap to host -------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_block_swap_round_trip_equals_a_block_copy(dtype):
    """Swapping blocks out to host slots and back in to other device blocks
    moves exactly what a device-to-device copy of the same blocks would; no
    other byte of either pool changes."""
    rng = np.random.default_rng(60)
    nb, nkv, B, d, H = 12, 2, 4, 8, 5
    k, v = _pools(nb, nkv, B, d, rng, dtype)
    hk, hv = _pools(H, nkv, B, d, rng, dtype)
    out_pairs = np.array([[3, 0], [7, 4], [2, 1]], np.int32)
    k1, v1, hk1, hv1 = oracle.block_swap(k, v, hk, hv, out_pairs, oracle.SWAP_OUT)
    assert np.array_equal(k1, k) and np.array_equal(v1, v)      # the source is untouched
    for src, dst in out_pairs:
        assert np.array_equal(hk1[dst], k[src]) and np.array_equal(hv1[dst], v[src])
    untouched = [h for h in range(H) if h not in out_pairs[:, 1]]
    assert np.array_equal(hk1[untouched], hk[untouched])
    in_pairs = np.array([[0, 9], [4, 10], [1, 11]], np.int32)
    k2, v2, hk2, hv2 = oracle.block_swap(k1, v1, hk1, hv1, in_pairs, oracle.SWAP_IN)
    kc, vc = oracle.block_copy(k, v, np.array([[3, 9], [7, 10], [2, 11]], np.int32))
    assert np.array_equal(k2, kc) and np.array_equal(v2, vc)
    assert np.array_equal(hk2, hk1) and np.array_equal(hv2, hv1)


def test_block_swap_rejects_out_of_range_pairs():
    rng = np.random.default_rng(61)
    k, v = _pools(4, 1, 4, 8, rng)
    hk, hv = _pools(2, 1, 4, 8, rng)
    with pytest.raises(oracle.OracleError):
        oracle.block_swap(k, v, hk, hv, np.array([[0, 2]], np.int32), oracle.SWAP_OUT)
    with pytest.raises(oracle.OracleError):
        oracle.block_swap(k, v, hk, hv, np.array([[2, 0]], np.int32), oracle.SWAP_IN)


# --- multi-token (extend) attention ---------------------------------------------------
def _extend_case(rng, lens, ns, nb=40, nkv=2, Hq=4, B=4, d=8, dtype="f32"):
    k, v = _pools(nb, nkv, B, d, rng, dtype)
    S = len(lens)
    width = max(-(-L // B) for L in lens)
    tables = np.stack([rng.permutation(nb)[:width] for _ in range(S)]).astype(np.int32)
    q_start = np.concatenate([[0], np.cumsum(ns)]).astype(np.int32)
    q = rng.standard_normal((int(q_start[-1]), Hq, d)).astype(np.float32)
    if dtype == "bf16":
        q = f32_to_bf16_bits(q)
    return k, v, q, q_start, tables, np.array(lens, np.int32)


def test_extend_with_one_query_per_sequence_is_decode():
    """One new token per sequence sits at position L - 1 and sees the whole
    context: the extend oracle must equal the decode oracle bit for bit."""
    rng = np.random.default_rng(70)
    k, v, q, qs, tables, lens = _extend_case(rng, [5, 17, 1, 40], [1, 1, 1, 1])
    ext = oracle.extend(k, v, q, qs, tables, lens, 0.3)
    dec = oracle.decode(k, v, q, tables, lens, 0.3)
    assert np.array_equal(ext, dec)


def test_extend_equal_keys_give_causal_means():
    """All keys zero: query j of a sequence averages V over tokens 0..p_j,
    p_j = L - n + j -- a different prefix for every query."""
    rng = np.random.default_rng(71)
    k, v, q, qs, tables, lens = _extend_case(rng, [13, 9], [5, 9])
    k[...] = 0
    out = oracle.extend(k, v, q, qs, tables, lens, 1.0)
    B = 4
    for s in range(2):
        n, L = qs[s + 1] - qs[s], lens[s]
        Kc, Vc = oracle.gather(k, v, tables[s], 1, L)
        for j in range(n):
            p = L - n + j
            assert np.allclose(out[qs[s] + j, 2:4], Vc[:p + 1].mean(axis=0), rtol=0, atol=1e-12)


def test_extend_is_blind_to_tokens_after_each_position():
    """Changing every token after position p changes no output of a query at
    p or before."""
    rng = np.random.default_rng(72)
    k, v, q, qs, tables, lens = _extend_case(rng, [21], [7], B=4)
    out = oracle.extend(k, v, q, qs, tables, lens, 0.5)
    L, n, B = 21, 7, 4
    p_cut = L - n + 3                          # query 3's position
    k2, v2 = k.copy(), v.copy()
    for t in range(p_cut + 1, L):              # overwrite the later tokens
        b, r = tables[0, t // B], t % B
        k2[b, :, r, :] = 1e3
        v2[b, :, :, r] = -1e3
    out2 = oracle.extend(k2, v2, q, qs, tables, lens, 0.5)
    assert np.array_equal(out[:4], out2[:4])
    assert not np.array_equal(out[4:], out2[4:])


def test_extend_chunks_compose():
    """Prefilling n tokens in one call equals two calls on consecutive chunks
    (the first with the context ending at the chunk boundary)."""
    rng = np.random.default_rng(73)
    k, v, q, qs, tables, lens = _extend_case(rng, [30], [12], dtype="bf16")
    whole = oracle.extend(k, v, q, qs, tables, lens, 0.4)
    first = oracle.extend(k, v, q[:5], np.array([0, 5], np.int32), tables,
                          np.array([23], np.int32), 0.4)
    second = oracle.extend(k, v, q[5:], np.array([0, 7], np.int32), tables, lens, 0.4)
    assert np.array_equal(whole, np.concatenate([first, second]))


def test_extend_rejects_more_queries_than_context():
    rng = np.random.default_rng(74)
    k, v, q, qs, tables, lens = _extend_case(rng, [3], [4])
    with pytest.raises(oracle.OracleError):
        oracle.extend(k, v, q, qs, tables, lens, 1.0)
