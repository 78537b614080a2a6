"""GPU parity for block sizes 8 and 32 (the vLLM post's "Where it bites":
bigger blocks mean fewer table entries but more waste in the last block,
smaller ones the reverse and more, smaller reads).  Decode on bf16 and 8-bit
pools against the oracle on every output; slot write and block copy
bit-exact.  The 16-token case is covered by the other GPU tests."""
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, block_copy_case, decode_case, kv_write_case
from workloads.gen import from_numpy_storage, to_numpy_storage

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def pk():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import paged_kv_cache_335_amd as pk
    return pk


def _small(key, B, dtype):
    base = {
        "llama2_7b_mha": dict(num_seqs=6, lengths=("uniform", 128, 700), pool=("fixed", 512 * 16 // B),
                     table_width=48 * 16 // B),
        "llama3_8b_gqa": dict(num_seqs=24, lengths=("lognormal", 256, 1.0, 16, 2048),
                     table_width=128 * 16 // B),
        "prefix_sharing": dict(num_seqs=16, prompts=4, lengths=("shared", 96, 1, 40),
                     table_width=9 * 16 // B + 1),
        "long_context_128k": dict(num_seqs=2, lengths=("fixed", 4096), pool=("fixed", 512 * 16 // B),
                     table_width=256 * 16 // B),
    }[key]
    return CONFIGS[key].scaled(block_size=B, dtype=dtype, **base)


@pytest.mark.parametrize("B", [8, 32])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("key", ["llama2_7b_mha", "llama3_8b_gqa", "prefix_sharing", "long_context_128k"])
def test_decode_block_sizes_all_elements(pk, key, dtype, B):
    cfg = _small(key, B, dtype)
    c = decode_case(cfg, payload="numpy", device="cuda")
    ref = oracle.decode(*c.oracle_inputs(), c.scale)
    for P in (0, 2 * B, 64 if B < 64 else B):
        out = pk.pa_decode(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens, c.scale,
                           partition_tokens=P)
        torch.cuda.synchronize()
        err = np.abs(out.float().cpu().numpy().astype(np.float64) - ref)
        _log(f"{key} {dtype} B={B} P={P}: max|err| {err.max():.3e}")
        assert np.isfinite(err).all() and err.max() <= 2e-2


@pytest.mark.parametrize("B", [8, 32])
def test_decode_block_sizes_odd_lengths_and_groups(pk, B):
    """Lengths around tile and block edges (a tile of 8-token blocks can end
    mid-range), group sizes 1 and 16."""
    for G, d in ((1, 128), (16, 64)):
        cfg = CONFIGS["llama3_8b_gqa"].scaled(num_seqs=12, num_q_heads=2 * G, num_kv_heads=2, head_dim=d,
                                     block_size=B, lengths=("uniform", 1, 300),
                                     table_width=300 // B + 2, seed=40 + B + G)
        c = decode_case(cfg, payload="numpy", device="cuda")
        ref = oracle.decode(*c.oracle_inputs(), c.scale)
        for P in (B, 3 * B, 0):
            out = pk.pa_decode(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens,
                               c.scale, partition_tokens=P)
            torch.cuda.synchronize()
            err = np.abs(out.float().cpu().numpy().astype(np.float64) - ref).max()
            assert err <= 2e-2, (G, d, P, err)


@pytest.mark.parametrize("B", [8, 32])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_kv_write_and_block_copy_block_sizes_bit_exact(pk, dtype, B):
    w = kv_write_case(100, 4, 128, B, 300, dtype=dtype, skip_fraction=0.1, seed=B)
    kref, vref = oracle.kv_write(w.k_pool, w.v_pool, w.k_new, w.v_new, w.slot_mapping)
    tdt = "u8" if dtype == "fp8" else dtype
    k = torch.from_numpy(w.k_pool).cuda() if dtype == "fp8" else \
        from_numpy_storage(w.k_pool, dtype, "cuda")
    v = torch.from_numpy(w.v_pool).cuda() if dtype == "fp8" else \
        from_numpy_storage(w.v_pool, dtype, "cuda")
    src = "bf16"
    pk.pa_kv_write(k, v, from_numpy_storage(w.k_new, src, "cuda"),
                   from_numpy_storage(w.v_new, src, "cuda"),
                   torch.from_numpy(w.slot_mapping).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(to_numpy_storage(k), kref), tdt
    assert np.array_equal(to_numpy_storage(v), vref)
    c = block_copy_case(200, 4, 128, B, 60, dtype=dtype, seed=B + 1)
    kref, vref = oracle.block_copy(c.k_pool, c.v_pool, c.pairs)
    k = torch.from_numpy(c.k_pool).cuda() if dtype == "fp8" else \
        from_numpy_storage(c.k_pool, dtype, "cuda")
    v = torch.from_numpy(c.v_pool).cuda() if dtype == "fp8" else \
        from_numpy_storage(c.v_pool, dtype, "cuda")
    pk.pa_block_copy(k, v, torch.from_numpy(c.pairs).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(to_numpy_storage(k), kref)
    assert np.array_equal(to_numpy_storage(v), vref)


@pytest.mark.slow
@pytest.mark.parametrize("B", [8, 32])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_decode_block_sizes_full_size_all_outputs(pk, dtype, B):
    """The 256-sequence GQA workload at full size with 8- and 32-token
    blocks, bf16 and 8-bit (regions side by side, as the runtime allocates
    them), in the benchmark's launch configuration: every output against
    the oracle, and a second call bit-identical."""
    cfg = CONFIGS["llama3_8b_gqa"].scaled(block_size=B, dtype=dtype, table_width=512 * 16 // B)
    _log(f"llama3_8b_gqa {dtype} B={B}: generating on the GPU")
    c = decode_case(cfg, payload="torch", device="cuda")
    k, v = c.k_pool, c.v_pool
    if dtype == "fp8":
        k, v = pk.fp8_pools_side_by_side(k, v, "cuda")
    got = pk.pa_decode(c.q, k, v, c.block_tables, c.context_lens, c.scale).clone()
    again = pk.pa_decode(c.q, k, v, c.block_tables, c.context_lens, c.scale)
    torch.cuda.synchronize()
    assert torch.equal(got, again)
    del k, v, again
    S, Hq = cfg.num_seqs, cfg.num_q_heads
    pairs = np.array([[s, h] for s in range(S) for h in range(Hq)], np.int32)
    _log(f"llama3_8b_gqa {dtype} B={B}: oracle over all {len(pairs)} outputs")
    ref = oracle.decode_pairs(*c.oracle_inputs(), c.scale, pairs)
    err = np.abs(got.float().cpu().numpy().astype(np.float64)[pairs[:, 0], pairs[:, 1]] - ref)
    _log(f"llama3_8b_gqa {dtype} B={B} full size: max|err| {err.max():.3e}")
    assert np.isfinite(err).all() and err.max() <= 2e-2
    del c
    torch.cuda.empty_cache()
