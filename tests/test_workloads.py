"""The seeded generators: deterministic, valid tables, poison where no
context lives, and the configured shapes.  CPU only."""
import numpy as np
import pytest

from workloads import (CONFIGS, POISON_K, POISON_V, block_copy_case, decode_case,
                       decode_structure, kv_write_case)
from workloads.gen import to_numpy_storage


def test_same_seed_same_bytes():
    cfg = CONFIGS["llama3_8b_gqa"].scaled(num_seqs=8, lengths=("lognormal", 128, 1.0, 16, 512),
                                 table_width=32)
    a, b = decode_case(cfg), decode_case(cfg)
    for x, y in zip(a.oracle_inputs(), b.oracle_inputs()):
        assert np.array_equal(x, y)
    c = decode_case(cfg, seed=99)
    assert not np.array_equal(a.oracle_inputs()[2], c.oracle_inputs()[2])


@pytest.mark.parametrize("key", ["tiny_f32", "llama2_7b_mha", "llama3_8b_gqa", "prefix_sharing", "prefix_sharing_cow", "long_context_128k"])
def test_full_size_structure(key):
    cfg = CONFIGS[key]
    lens, nb, tables, live = decode_structure(cfg)
    B = cfg.block_size
    assert lens.shape == (cfg.num_seqs,) and lens.min() >= 1
    assert tables.shape == (cfg.num_seqs, cfg.table_width)
    assert tables.min() >= 0 and tables.max() < nb
    nblk = (lens + B - 1) // B
    if cfg.lengths[0] != "shared":
        used = np.concatenate([tables[s, :nblk[s]] for s in range(cfg.num_seqs)])
        assert len(np.unique(used)) == len(used)       # no block used twice
    assert live.sum() == (lens.sum() if cfg.lengths[0] != "shared" else live.sum())
    if key == "long_context_128k":
        assert nb == 32768 and lens.sum() == 4 * 131072 and live.all()
    if key == "llama3_8b_gqa":
        assert lens.min() >= 16 and lens.max() <= 8192
        assert nb == int(np.ceil(1.1 * nblk.sum()))
    if key == "llama2_7b_mha":
        assert nb == 16384 and lens.min() >= 128 and lens.max() <= 2048
    if key.startswith("prefix_sharing"):
        shared = cfg.lengths[1] // B
        for p in range(cfg.prompts):
            rows = tables[p * cfg.samples:(p + 1) * cfg.samples, :shared]
            assert (rows == rows[0]).all()


def test_poison_fills_exactly_the_dead_slots():
    cfg = CONFIGS["tiny_f32"]
    c = decode_case(cfg)
    k, v = to_numpy_storage(c.k_pool), to_numpy_storage(c.v_pool)
    dead = ~c.live
    assert (k[dead.nonzero()[0], :, dead.nonzero()[1], :] == POISON_K).all()
    assert (v.transpose(0, 3, 1, 2)[dead] == POISON_V).all()
    assert not (k[c.live.nonzero()[0], :, c.live.nonzero()[1], :] == POISON_K).any()


def test_kv_write_and_copy_cases_are_valid():
    w = kv_write_case(64, 2, 16, 16, 300, skip_fraction=0.1, seed=3)
    s = w.slot_mapping[w.slot_mapping >= 0]
    assert len(np.unique(s)) == len(s) and s.max() < 64 * 16 and (w.slot_mapping == -1).any()
    c = block_copy_case(64, 2, 16, 16, 20, seed=4)
    src, dst = c.pairs[:, 0], c.pairs[:, 1]
    assert len(np.unique(dst)) == len(dst) and not set(dst) & set(src)
