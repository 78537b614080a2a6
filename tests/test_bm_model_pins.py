"""Pins for the block-manager reference model: the pages' worked allocation
examples, the waste bound, refcount and copy-on-write rules, and all-or-
nothing exhaustion.  CPU only."""
import json
import os
import random

import pytest

from oracle.bm_model import (EINVAL, ENOMEM, OK, BlockManagerModel, contiguous_reservation,
                             initial_free_stack, paged_accounting, splitmix64_stream)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def ex():
    return json.load(open(os.path.join(GOLDEN, "allocation_examples.json")))


def test_reserved_space_example(ex):
    e = ex["reserved_space"]
    acc = contiguous_reservation([e["used"]], e["reserved"])
    assert acc["empty"] == e["expected_empty"]
    assert round(100 * acc["wasted_fraction"]) == e["expected_wasted_percent_printed"]


def test_add_pages_example(ex):
    e = ex["add_pages"]
    m = BlockManagerModel(16, e["block_size"], seed=0)
    s = m.add_seq()
    st, slots, pairs = m.append(s, e["tokens"])
    assert st == OK and pairs == []
    _, table, n = m.block_table(s)
    assert len(table) == e["expected_pages"]
    stats = m.stats()
    assert stats["allocated_slots"] - stats["stored_tokens"] == e["expected_empty_slots"]
    # growing token by token gives the same pages: a page is added only when
    # the current one is full
    m2 = BlockManagerModel(16, e["block_size"], seed=0)
    s2 = m2.add_seq()
    pages_after = []
    for _ in range(e["tokens"]):
        m2.append(s2, 1)
        pages_after.append(len(m2.block_table(s2)[1]))
    assert pages_after == [1, 1, 1, 1, 2, 2, 2, 2, 3, 3, 3]
    assert m2.block_table(s2)[1] == table


def test_batch_memory_example(ex):
    e = ex["batch_memory"]
    cont = contiguous_reservation(e["lengths"], e["reserve_per_request"])
    paged = paged_accounting(e["lengths"], e["block_size"])
    assert cont["reserved"] == e["expected_contiguous"]
    assert paged["slots"] == e["expected_paged"]
    assert paged["stored"] == e["expected_stored"]
    assert round(100 * (1 - paged["slots"] / cont["reserved"])) == \
        e["expected_saving_percent_printed"]
    # the manager itself reaches the same numbers
    m = BlockManagerModel(64, e["block_size"], seed=7)
    for L in e["lengths"]:
        s = m.add_seq()
        assert m.append(s, L)[0] == OK
    st = m.stats()
    assert st["allocated_slots"] == e["expected_paged"]
    assert st["stored_tokens"] == e["expected_stored"]


def test_share_prefixes_example(ex):
    e = ex["share_prefixes"]
    B = e["block_size"]
    m = BlockManagerModel(32, B, seed=3)
    a = m.add_seq()
    m.append(a, e["shared_blocks"] * B)
    st, b = m.fork(a)
    assert st == OK
    stats = m.stats()
    assert stats["shared_blocks"] == e["shared_blocks"]
    assert all(m.refcount[x] == e["expected_refcount"] for x in m.block_table(a)[1])
    assert stats["logical_blocks"] - stats["used_blocks"] == e["expected_copies_avoided"]
    # growing past a full shared block: a fresh block, no copy
    for s in (a, b):
        st, slots, pairs = m.append(s, 2)
        assert st == OK and pairs == []
    assert m.stats()["cow_copies"] == e["expected_cow_copies_after_append"]
    ta, tb = m.block_table(a)[1], m.block_table(b)[1]
    assert ta[:3] == tb[:3] and ta[3] != tb[3]


@pytest.mark.parametrize("n", [2, 4, 5])
def test_partial_shared_tail_copies_n_minus_one(n):
    """Writing into a shared, partly filled tail block takes a private copy;
    the last holder writes in place, so n sharers make n - 1 copies."""
    B = 4
    m = BlockManagerModel(64, B, seed=11)
    p = m.add_seq()
    m.append(p, 3 * B + 2)
    kids = [m.fork(p)[1] for _ in range(n - 1)]
    tail = m.block_table(p)[1][-1]
    all_pairs = []
    for s in [p] + kids:
        st, slots, pairs = m.append(s, 1)
        assert st == OK
        all_pairs += pairs
        # the new token lands at offset 2 of whatever tail block s now holds
        assert slots == [m.block_table(s)[1][-1] * B + 2]
    assert len(all_pairs) == n - 1
    assert all(src == tail for src, _ in all_pairs)
    assert m.refcount[tail] == 1
    assert m.stats()["cow_copies"] == n - 1
    tails = {m.block_table(s)[1][-1] for s in [p] + kids}
    assert len(tails) == n


def test_full_shared_tail_needs_no_copy():
    B = 4
    m = BlockManagerModel(64, B, seed=12)
    p = m.add_seq()
    m.append(p, 4 * B)
    kids = [m.fork(p)[1] for _ in range(3)]
    for s in [p] + kids:
        st, slots, pairs = m.append(s, 1)
        assert st == OK and pairs == []
    assert m.stats()["cow_copies"] == 0


def test_exhaustion_is_all_or_nothing():
    B = 4
    m = BlockManagerModel(5, B, seed=13)
    s = m.add_seq()
    assert m.append(s, 17)[0] == OK          # 5 blocks, 3 slots free in the tail
    before = (list(m.free), list(m.refcount), m.block_table(s), m.stats())
    st, slots, pairs = m.append(s, 4)        # needs one more block
    assert st == ENOMEM and slots == [] and pairs == []
    after = (list(m.free), list(m.refcount), m.block_table(s), m.stats())
    assert before[:3] == after[:3]
    assert after[3]["enomem_events"] == 1
    assert m.append(s, 3)[0] == OK           # fits exactly


def test_copy_on_write_counts_toward_exhaustion():
    B = 4
    m = BlockManagerModel(3, B, seed=0)
    p = m.add_seq()
    m.append(p, 6)                           # 2 blocks used, 1 free
    c = m.fork(p)[1]
    assert m.append(c, 3)[0] == ENOMEM       # a copy and a new block: two needed, one free
    assert m.append(c, 2)[0] == OK           # the copy takes the last block
    assert m.append(p, 2)[0] == OK           # p holds its tail alone now: in place
    assert m.append(p, 1)[0] == ENOMEM       # the next token needs a new block


def test_free_returns_blocks_and_rejects_bad_ids():
    m = BlockManagerModel(8, 4, seed=5)
    a = m.add_seq()
    m.append(a, 9)
    table = m.block_table(a)[1]
    free_before = list(m.free)
    assert m.free_seq(a) == OK
    assert m.free == free_before + table[::-1]
    assert m.free_seq(a) == EINVAL
    assert m.append(a, 1)[0] == EINVAL
    assert m.fork(a)[0] == EINVAL
    assert m.append(99, 1)[0] == EINVAL
    assert m.stats()["used_blocks"] == 0


def _check_invariants(m: BlockManagerModel):
    B = m.B
    counts = [0] * m.num_blocks
    for seq in m.seqs:
        if not seq.alive:
            continue
        assert len(seq.table) == -(-seq.n_tokens // B)
        assert len(set(seq.table)) == len(seq.table)
        for b in seq.table:
            counts[b] += 1
    assert counts == m.refcount
    free = set(m.free)
    assert len(free) == len(m.free)
    used = {b for b in range(m.num_blocks) if m.refcount[b] > 0}
    assert free.isdisjoint(used) and free | used == set(range(m.num_blocks))
    st = m.stats()
    # waste: fewer than B idle slots per live sequence (only tails are partial)
    assert st["allocated_slots"] - st["stored_tokens"] < B * max(1, st["live_seqs"])


def test_random_operations_keep_invariants():
    rnd = random.Random(2024)
    m = BlockManagerModel(200, 16, seed=99)
    live = []
    for step in range(3000):
        op = rnd.random()
        if op < 0.15 or not live:
            live.append(m.add_seq())
        elif op < 0.25:
            st, c = m.fork(rnd.choice(live))
            if st == OK:
                live.append(c)
        elif op < 0.35:
            s = rnd.choice(live)
            assert m.free_seq(s) == OK
            live.remove(s)
        else:
            s = rnd.choice(live)
            n_before = m.block_table(s)[2]
            st, slots, pairs = m.append(s, rnd.randint(0, 40))
            if st == OK:
                table = m.block_table(s)[1]
                for i, slot in enumerate(slots):
                    p = n_before + i
                    assert slot == table[p // 16] * 16 + p % 16
        _check_invariants(m)


def test_splitmix64_reference_values():
    """First outputs of SplitMix64 seeded with 0 and 1234567 (published test
    values of the generator)."""
    g = splitmix64_stream(1234567)
    assert [next(g) for _ in range(3)] == [6457827717110365317, 3203168211198807973,
                                          9817491932198370423]
    g0 = splitmix64_stream(0)
    assert next(g0) == 0xE220A8397B1DCDAF


def test_free_stack_is_a_permutation_and_seed_zero_pops_in_order():
    a = initial_free_stack(10, 0)
    assert a == list(range(9, -1, -1))
    m = BlockManagerModel(10, 4, seed=0)
    s = m.add_seq()
    m.append(s, 12)
    assert m.block_table(s)[1] == [0, 1, 2]
    b = initial_free_stack(1000, 42)
    assert sorted(b) == list(range(1000)) and b != list(range(999, -1, -1))


def test_swap_rules_by_hand():
    """Swap to a host pool, worked out from the stated rules: pool of 6
    unshuffled blocks (pops 0, 1, 2, ...), 4 host blocks (pops 0, 1, ...),
    block size 4."""
    m = BlockManagerModel(6, 4, 0)
    assert m.set_host_blocks(4) == OK
    a = m.add_seq()
    assert m.append(a, 10)[0] == OK              # blocks 0, 1, 2
    st, b = m.fork(a)                            # shares all three
    assert st == OK
    st, pairs = m.swap_out(a)
    assert st == OK and pairs == [(0, 0), (1, 1), (2, 2)]
    assert m.refcount[:3] == [1, 1, 1]           # b still holds them: none freed
    assert m.free == [5, 4, 3] and m.host_free == [3]
    assert m.append(a, 1)[0] == EINVAL           # swapped: no appends, no forks
    assert m.fork(a)[0] == EINVAL
    assert m.swap_out(b) == (ENOMEM, [])         # 3 entries, 1 free host block
    assert m.free_seq(b) == OK                   # pushes 2, 1, 0
    assert m.free == [5, 4, 3, 2, 1, 0]
    st, pairs = m.swap_in(a)                     # pops 0, 1, 2 again
    assert st == OK and pairs == [(0, 0), (1, 1), (2, 2)]
    assert m.host_free == [3, 2, 1, 0] and m.seqs[a].table == [0, 1, 2]
    assert m.swap_in(a) == (EINVAL, [])
    s = m.stats()
    assert (s["swapped_out_blocks"], s["swapped_in_blocks"], s["swapped_seqs"]) == (3, 3, 0)
    # a swapped sequence that is freed returns its host blocks
    assert m.swap_out(a)[0] == OK and m.host_free == [3]
    assert m.free_seq(a) == OK and m.host_free == [3, 2, 1, 0]
    assert m.free == [5, 4, 3, 2, 1, 0]
    assert m.set_host_blocks(2) == OK and m.host_free == [1, 0]


def test_swap_out_then_in_restores_the_tokens_table_shape():
    """After swapping out and back in, a sequence has the same number of
    blocks and tokens, and appends continue from where it stopped."""
    m = BlockManagerModel(50, 16, 7)
    m.set_host_blocks(20)
    s = m.add_seq()
    m.append(s, 37)
    before = (len(m.seqs[s].table), m.seqs[s].n_tokens)
    assert m.swap_out(s)[0] == OK and m.swap_in(s)[0] == OK
    assert (len(m.seqs[s].table), m.seqs[s].n_tokens) == before
    st, slots, pairs = m.append(s, 1)
    assert st == OK and slots == [m.seqs[s].table[2] * 16 + 5] and pairs == []
