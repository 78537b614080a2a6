#!/usr/bin/env python3
"""Benchmark one decode step of a paged KV cache on one MI355X.

Workload (default): Llama-3-8B-shape GQA layer decode -- 256 sequences,
32 query heads over 8 KV heads, head dim 128, bf16, 16-token blocks,
context lengths lognormal (median 1024, sigma 1) clipped to [16, 8192], a
shuffled pool sized to the blocks needed plus 10%.

With --kv fp8 the same workload runs on an 8-bit cache (E4M3 codes with one
bf16 scale per token and kv head; queries and new tokens stay bf16).

With --config prefix_sharing (or prefix_sharing_cow) 64 prompts are written
once and forked into 4 samples each, which share the prompt's blocks (the
copy-on-write variant's partly filled shared tail is copied on the first
private append).  `value` counts every sequence's context (logical bytes);
the roofline uses the distinct token slots read (a shared prefix once),
since repeated reads of shared blocks can hit in the caches.

One step = the whole hot path for one batch: the host block manager appends
one token to every sequence (slots, new blocks, copy-on-write decisions), one
packed host-to-device metadata copy, the device table update, the slot write
of the 256 new tokens, and paged decode attention over every context.

Prints one JSON line.  `value` is KV bytes read per step / step time (GB/s);
`roofline` reports the decode kernel (HIP events on its stream) against the
8 TB/s HBM peak; `cpu_baseline` times the CPU oracle on a bounded sample of
the same batch.
"""
import argparse
import gc
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention: KV bytes read GB/s (% HBM peak) + decode tokens/s"
HBM_PEAK_GBPS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "decode_llama3_8b_gqa_hbm_traffic.md")
DECODE_SOURCES = ("paged_kv_cache_335_amd/csrc/pa_decode.hip",
                  "paged_kv_cache_335_amd/csrc/pa_device.h",
                  "paged_kv_cache_335_amd/csrc/pa_internal.h")


def measured_traffic(kv_bytes):
    """HBM bytes per decode launch from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE passes, scaled by a plain copy's counters), or
    None when the decode sources changed since the counters were taken or this
    run's workload is not the one they were taken on."""
    import hashlib
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    fields = dict(ln.split(": ", 1) for ln in text.splitlines()
                  if ln.startswith(("traffic_bytes_per_launch:", "algorithmic_bytes_per_launch:",
                                    "decode_source_sha256:")))
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if fields.get("decode_source_sha256") != h.hexdigest():
        return None
    if int(fields.get("algorithmic_bytes_per_launch", -1)) != int(kv_bytes):
        return None
    return int(fields["traffic_bytes_per_launch"])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="llama3_8b_gqa",
                    choices=["llama2_7b_mha", "llama3_8b_gqa", "prefix_sharing",
                             "prefix_sharing_cow", "long_context_128k"])
    ap.add_argument("--partition", type=int, default=0, help="partition tokens (0: library)")
    ap.add_argument("--block-size", type=int, default=16, choices=[8, 16, 32],
                    help="tokens per block (the table/tail-waste trade-off)")
    ap.add_argument("--mode", default="decode", choices=["decode", "extend"],
                    help="decode (default) or extend: chunked prefill over paged prefixes")
    ap.add_argument("--extend-seqs", type=int, default=32)
    ap.add_argument("--chunk", type=int, default=256, help="new tokens per sequence per step")
    ap.add_argument("--no-share", action="store_true",
                    help="prefix-sharing configs: read shared blocks once per sequence, not "
                         "once per prefix group")
    ap.add_argument("--kv", default="bf16", choices=["bf16", "fp8"],
                    help="cache storage: bf16, or 8-bit E4M3 codes + per-token scales")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-iters", type=int, default=10)
    ap.add_argument("--swap-blocks", type=int, default=1024,
                    help="after timing, swap this many resident blocks out to pinned host memory "
                         "and back, timed (0: skip)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after timing, run one plain device-to-device copy of this many MiB "
                         "(a kernel of known traffic, to scale the HBM byte counters)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    import paged_kv_cache_335_amd as pk
    from paged_kv_cache_335_amd.runtime import DeviceEvent, PagedKVCache
    from workloads import CONFIGS, draw_lengths
    from workloads.gen import unique_blocks

    if args.mode == "extend":
        return bench_extend(args, pk, DeviceEvent, PagedKVCache, CONFIGS, draw_lengths)

    cfg = CONFIGS[args.config]
    if args.block_size != cfg.block_size:
        cfg = cfg.scaled(block_size=args.block_size)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(dev)
    torch.cuda.set_stream(stream)
    S, Hq, Hkv, d, B = cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    W, K = args.warmup, args.steps
    steps = W + K

    rng = np.random.default_rng(cfg.seed)
    lens0 = draw_lengths(cfg, rng)           # context length at the first step
    # prefix sharing: prompts x samples sequences; each prompt's first
    # `shared` tokens are written once and shared by its samples (forks)
    shared = int(cfg.lengths[1]) if cfg.lengths[0] == "shared" else 0
    final = lens0.astype(np.int64) + steps
    need_blocks = unique_blocks(cfg, final) if shared else int(((final + B - 1) // B).sum())
    num_blocks = int(math.ceil(1.1 * need_blocks)) if cfg.pool[0] == "plus" else max(
        int(cfg.pool[1]), need_blocks)
    width = int((final.max() + B - 1) // B)
    log(f"{cfg.key}: S={S} Hq={Hq} Hkv={Hkv} d={d} sum L={int(lens0.sum())} "
        f"pool={num_blocks} blocks width={width}")

    fp8 = args.kv == "fp8"
    share = bool(shared) and not args.no_share
    cache = PagedKVCache(num_blocks, Hkv, d, S, width, block_size=B, shuffle_seed=cfg.seed,
                         dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev,
                         share_prefixes=share, max_group=max(1, 16 // (Hq // Hkv)))
    g = torch.Generator(device=dev)
    g.manual_seed(cfg.seed)
    if shared:
        # each prompt's shared tokens once, then its forks (so a prompt's
        # samples take adjacent table rows)
        log(f"prefill {cfg.prompts} prompts x {shared} shared tokens, {cfg.samples} samples each")
        seq_list = []
        for _ in range(cfg.prompts):
            s0 = cache.add_sequence()
            kn = torch.randn((shared, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
            vn = torch.randn((shared, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
            cache.append(np.array([s0], np.int32), np.array([shared], np.int32), kn, vn,
                         stream=stream)
            seq_list += [s0] + [cache.fork(s0) for _ in range(cfg.samples - 1)]
        seqs = np.array(seq_list, dtype=np.int32)
    else:
        seqs = np.array([cache.add_sequence() for _ in range(S)], dtype=np.int32)

    # prefill: every context token but the one each first step appends (past
    # the shared prefix, which is already in place)
    pre = (lens0 - 1 - shared).astype(np.int32)
    log(f"prefill {int(pre.sum())} tokens through the slot write")
    chunk = 16384
    start = 0
    order = np.arange(S)
    while start < S:
        # batches of whole sequences, about `chunk` tokens each
        tot, end = 0, start
        while end < S and (tot == 0 or tot + pre[end] <= chunk):
            tot += int(pre[end])
            end += 1
        kn = torch.randn((tot, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
        vn = torch.randn((tot, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
        cache.append(seqs[order[start:end]], pre[start:end], kn, vn, stream=stream)
        start = end
    torch.cuda.synchronize()

    # per-step inputs, drawn before timing
    qs = [torch.randn((S, Hq, d), generator=g, device=dev).to(torch.bfloat16) for _ in range(steps)]
    kns = [torch.randn((S, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
           for _ in range(steps)]
    vns = [torch.randn((S, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
           for _ in range(steps)]
    out = torch.empty((S, Hq, d), dtype=torch.bfloat16, device=dev)
    ones = np.ones(S, np.int32)
    P = cache.partition_tokens(Hq, args.partition)
    cache.workspace(Hq, args.partition)
    # bytes of one token's K and V rows for every kv head (8-bit: d codes and
    # one bf16 scale per side)
    kv_per_token = 2 * Hkv * (d + 2 if fp8 else d * 2)

    step_bytes = []
    step_unique = []  # bytes of distinct token slots read (a shared prefix counts once)
    base = (shared // B) * B  # tokens of each prompt's shared full blocks

    def unique_tokens(lens):
        lens = lens.astype(np.int64)
        return int(cfg.prompts * base + (lens - base).sum()) if shared else int(lens.sum())

    def step(i):
        cache.append(seqs, ones, kns[i], vns[i], stream=stream)
        cache.decode(qs[i], out=out, partition_tokens=args.partition, stream=stream)

    # Python's cyclic garbage collector: a full collection takes tens of
    # milliseconds in this process and, when one fell inside the timed steps,
    # left the GPU idle for a few steps' worth of time.  Collect before the
    # warm-up (whose steps then also warm the host path) and keep it off
    # until the timed steps and the roofline calls have run.
    gc.collect()
    gc.disable()
    log(f"warmup {W} steps (partition {P} tokens)")
    for i in range(W):
        step(i)
        step_bytes.append(int(cache.host_lens[:S].sum()) * kv_per_token)
        step_unique.append(unique_tokens(cache.host_lens[:S]) * kv_per_token)
    torch.cuda.synchronize()
    # the timed steps carry no events: recording one leaves the GPU idle for
    # a few microseconds before the next kernel, which is instrumentation,
    # not part of the path
    log(f"timing {K} steps")
    t0 = time.perf_counter()
    for i in range(W, steps):
        step(i)
        step_bytes.append(int(cache.host_lens[:S].sum()) * kv_per_token)
        step_unique.append(unique_tokens(cache.host_lens[:S]) * kv_per_token)
    t_enq = time.perf_counter()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    host_ms = (t_enq - t0) * 1e3 / K
    ms_step = (t1 - t0) * 1e3 / K
    timed_bytes = step_bytes[W:]
    kv_avg = float(np.mean(timed_bytes))
    value = kv_avg / (ms_step * 1e-3) / 1e9

    # decode duration for the roofline: K decode calls back to back on the
    # same stream, over the last step's batch, between two fence-free HIP
    # events (each call = the decode kernel and its reduce kernel)
    ea, eb = DeviceEvent(timing=True), DeviceEvent(timing=True)
    ea.record(stream)
    for _ in range(K):
        cache.decode(qs[-1], out=out, partition_tokens=args.partition, stream=stream)
    eb.record(stream)
    eb.synchronize()
    gc.enable()  # off since before the warm-up
    dec_ms_avg = ea.elapsed_ms(eb) / K
    last_bytes = step_bytes[-1]
    dec_gbps = last_bytes / (dec_ms_avg * 1e-3) / 1e9
    # with a shared prefix, the bytes that must come from HBM are the
    # distinct slots; repeated reads of shared blocks can hit in the caches
    dec_gbps_unique = step_unique[-1] / (dec_ms_avg * 1e-3) / 1e9
    log(f"step {ms_step:.3f} ms ({value:.0f} GB/s); decode {dec_ms_avg * 1e3:.1f} us "
        f"({dec_gbps:.0f} GB/s); host enqueue {host_ms:.3f} ms/step")

    # cold decode: caches flushed before each call (outside the event window)
    cold = None
    if args.cold_iters > 0:
        flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
        cold_ms = []
        for _ in range(args.cold_iters):
            flush.fill_(1.0)
            a, b = DeviceEvent(timing=True), DeviceEvent(timing=True)
            a.record(stream)
            cache.decode(qs[-1], out=out, partition_tokens=args.partition, stream=stream)
            b.record(stream)
            b.synchronize()
            cold_ms.append(a.elapsed_ms(b))
        del flush
        cold = {"us_mean": float(np.mean(cold_ms)) * 1e3, "us_min": float(np.min(cold_ms)) * 1e3,
                "GBps": step_bytes[-1] / (np.mean(cold_ms) * 1e-3) / 1e9}
        log(f"cold decode {cold['us_mean']:.1f} us ({cold['GBps']:.0f} GB/s)")

    # the last step's output again, for the sampled parity check below
    cache.decode(qs[-1], out=out, partition_tokens=args.partition, stream=stream)
    torch.cuda.synchronize()

    copy_write = copy_write_probe(pk, cache, kns[-1], vns[-1], stream)

    swap = None
    if args.swap_blocks > 0:
        swap = swap_probe(pk, cache, args.swap_blocks, stream)

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * 1024 * 1024 // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: {args.copy_probe_mib} MiB read + {args.copy_probe_mib} MiB written")
        del src, dst

    lens_now = cache.host_lens[:S].copy()
    stats = cache.bm.stats()
    tail_waste = 100.0 * (stats["allocated_slots"] - stats["stored_tokens"]) / max(
        1, stats["allocated_slots"])
    contiguous_util = 100.0 * float(lens_now.sum()) / (S * int(final.max()))

    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8e4m3 kv, bf16 mfma" if fp8 else "bf16", "data": "synthetic",
        "config": {
            "workload": f"{cfg.key}: {cfg.description}" + (
                "; 8-bit cache (E4M3 + per-token bf16 scales)" if fp8 else ""),
            "kv_storage": args.kv,
            "num_seqs": S, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": d,
            "block_size": B, "pool_blocks": num_blocks, "partition_tokens": P,
            "mean_context_tokens": round(float(lens_now.mean()), 1),
            "kv_bytes_per_step": int(kv_avg),
            "kv_bytes_unique_per_step": int(np.mean(step_unique[W:])),
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "tokens_per_s": round(S / (ms_step * 1e-3), 1),
        "host_enqueue_ms_per_step": round(host_ms, 4),
        "decode": {"us_mean": round(dec_ms_avg * 1e3, 2), "GBps": round(dec_gbps, 1),
                   "kv_bytes": int(last_bytes), "calls": K,
                   "tokens_per_s": round(S / (dec_ms_avg * 1e-3), 1),
                   "GBps_unique": round(dec_gbps_unique, 1),
                   "kv_bytes_unique": int(step_unique[-1])},
        "decode_cold": cold,
        "roofline": {"bound": "hbm", "achieved": round(dec_gbps_unique, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(dec_gbps_unique / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(kv_avg)
                     if args.partition == 0 and not fp8 else None},
        "cache_ops": copy_write,
        "block_swap": swap,
        "block_manager": {"tail_waste_pct": round(tail_waste, 3),
                          "contiguous_reservation_utilisation_pct": round(contiguous_util, 2),
                          "cow_copies": stats["cow_copies"]},
        "pages_context_no_hardware_given": {
            "prior_systems_kv_utilisation": "20-40%", "paging_waste": "under 4%",
            "vllm_throughput_vs_prior": "2-4x"},
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"], result["parity_sample"] = cpu_baseline(
            cache, qs[-1], out, lens_now, S, Hq, d, kv_per_token, args.cpu_seconds)

    print(json.dumps(result), flush=True)


MFMA_BF16_PEAK_TFLOPS = 2500.0


def bench_extend(args, pk, DeviceEvent, PagedKVCache, CONFIGS, draw_lengths):
    """Chunked prefill: `extend_seqs` sequences with cached prefixes drawn like
    the decode workload's lengths; every step appends `chunk` new tokens to
    each (block manager, slot write) and runs causal attention of those
    queries over the whole paged context.  Reports attention TFLOP/s against
    the bf16 MFMA peak (the path is matrix-bound at these chunk sizes)."""
    cfg = CONFIGS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(dev)
    torch.cuda.set_stream(stream)
    S, Hq, Hkv, d, B = (args.extend_seqs, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                        cfg.block_size)
    W, K, C = args.warmup, args.steps, args.chunk
    rng = np.random.default_rng(cfg.seed)
    lens0 = draw_lengths(cfg, rng)[:S].astype(np.int64)
    final = lens0 + (W + K) * C
    need = int(((final + B - 1) // B).sum())
    num_blocks = int(math.ceil(1.1 * need))
    width = int((final.max() + B - 1) // B)
    cache = PagedKVCache(num_blocks, Hkv, d, S, width, block_size=B, shuffle_seed=cfg.seed,
                         device=dev)
    seqs = np.array([cache.add_sequence() for _ in range(S)], dtype=np.int32)
    g = torch.Generator(device=dev)
    g.manual_seed(cfg.seed)
    log(f"extend: S={S} chunk={C} prefix sum={int(lens0.sum())} pool={num_blocks} blocks")
    for i in range(S):  # prefixes through the slot write
        n = int(lens0[i])
        kn = torch.randn((n, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
        vn = torch.randn((n, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
        cache.append(seqs[i:i + 1], np.array([n], np.int32), kn, vn, stream=stream)
    torch.cuda.synchronize()
    steps = W + K
    T = S * C
    qs = [torch.randn((T, Hq, d), generator=g, device=dev).to(torch.bfloat16) for _ in range(steps)]
    kns = [torch.randn((T, Hkv, d), generator=g, device=dev).to(torch.bfloat16) for _ in range(steps)]
    vns = [torch.randn((T, Hkv, d), generator=g, device=dev).to(torch.bfloat16) for _ in range(steps)]
    out = torch.empty((T, Hq, d), dtype=torch.bfloat16, device=dev)
    ns = np.full(S, C, np.int32)
    flops, kv_bytes = [], []
    ev = [(DeviceEvent(timing=True), DeviceEvent(timing=True)) for _ in range(steps)]
    scale = d ** -0.5
    q_start = torch.from_numpy(np.arange(S + 1, dtype=np.int32) * C).to(dev)

    def step(i):
        cache.append(seqs, ns, kns[i], vns[i], stream=stream)
        tables, lens = cache.bm.export(seqs, width, pad_block=0)
        d_tables = torch.from_numpy(tables).to(dev, non_blocking=False)
        d_lens = torch.from_numpy(lens).to(dev, non_blocking=False)
        ev[i][0].record(stream)
        pk.pa_extend(qs[i], cache.k_pool, cache.v_pool, q_start, d_tables, d_lens, scale,
                     out=out, stream=stream)
        ev[i][1].record(stream)
        L = lens.astype(np.int64)
        # sum over queries of (position + 1): query j of a sequence sees L - C + j + 1 tokens
        seen = (C * (L - C) + C * (C + 1) // 2).sum()
        flops.append(int(seen) * Hq * 4 * d)
        kv_bytes.append(int(L.sum()) * 2 * Hkv * d * 2)

    gc.collect()  # no collector pause inside the timed steps (as for decode)
    gc.disable()
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(W, steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gc.enable()
    ms_step = (t1 - t0) * 1e3 / K
    ext_ms = [ev[i][0].elapsed_ms(ev[i][1]) for i in range(W, steps)]
    ext_avg = float(np.mean(ext_ms))
    fl = float(np.mean(flops[W:]))
    tflops = fl / (ext_avg * 1e-3) / 1e12
    log(f"extend step {ms_step:.3f} ms; attention {ext_avg * 1e3:.1f} us, {tflops:.1f} TFLOP/s")
    result = {
        "metric": "paged extend (chunked prefill) attention: TFLOP/s + query tokens/s",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{cfg.key} shape, {S} sequences with cached prefixes, "
                               f"{C}-token chunks", "num_seqs": S, "chunk": C,
                   "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": d, "block_size": B,
                   "mean_context_tokens": round(float(np.mean(lens0)) + (W + K) * C / 2, 1)},
        "extend": {"us_mean": round(ext_avg * 1e3, 2), "us_min": round(min(ext_ms) * 1e3, 2),
                   "query_tokens_per_s": round(T / (ext_avg * 1e-3), 1),
                   "kv_GBps_unique": round(float(np.mean(kv_bytes[W:])) / (ext_avg * 1e-3) / 1e9, 1)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None},
    }
    if not args.no_cpu_baseline:
        tables, lens = cache.bm.export(seqs, width, pad_block=0)
        result["cpu_baseline"], result["parity_sample"] = extend_cpu_baseline(
            cache, qs[-1], out, tables, lens, C, Hq, d, scale, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def extend_cpu_baseline(cache, q, out, tables, lens, C, Hq, d, scale, seconds):
    """Time the CPU oracle's extend (as it stands) on whole sequences of the
    last timed step's batch: one sequence first, then as many as fit in about
    `seconds` of CPU work (in a fixed order).  Also compares the sampled rows
    with the GPU's."""
    import oracle
    from workloads.gen import to_numpy_storage
    log("cpu baseline (extend): copying the pool to the host")
    k = to_numpy_storage(cache.k_pool)
    v = to_numpy_storage(cache.v_pool)
    qn = to_numpy_storage(q)
    got_all = out.float().cpu().numpy().astype(np.float64)
    lens = lens.astype(np.int32)
    threads = oracle.max_threads()

    def run(sel):
        sel = np.asarray(sel)
        rows = (sel[:, None] * C + np.arange(C)[None, :]).reshape(-1)
        q_start = (np.arange(len(sel) + 1) * C).astype(np.int32)
        t = time.perf_counter()
        ref = oracle.extend(k, v, np.ascontiguousarray(qn[rows]), q_start,
                            np.ascontiguousarray(tables[sel]), np.ascontiguousarray(lens[sel]),
                            scale)
        return time.perf_counter() - t, ref, rows

    def flops_of(sel):
        L = lens[np.asarray(sel)].astype(np.int64)
        return int((C * (L - C) + C * (C + 1) // 2).sum()) * Hq * 4 * d

    order = np.random.default_rng(0).permutation(len(lens))
    t1, _, _ = run(order[:1])
    n = int(max(1, min(len(lens), seconds // max(t1, 1e-3))))
    sel = order[:n]
    dt, ref, rows = run(sel)
    err = float(np.abs(got_all[rows] - ref).max())
    fl = flops_of(sel)
    log(f"cpu baseline (extend): {n} sequences x {C} queries on {threads} threads, {dt:.2f} s, "
        f"{fl / dt / 1e12:.4f} TFLOP/s; sampled parity max|err| {err:.3e}")
    base = {"value": round(fl / dt / 1e12, 5), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{n} of {len(lens)} sequences of the last timed step's batch, all {C} "
                      f"queries and {Hq} query heads each ({dt:.1f} s); fp64 C oracle, OpenMP",
            "seconds": round(dt, 3), "query_tokens_per_s": round(n * C / dt, 2)}
    return base, {"rows": int(len(rows)), "max_abs_err": err, "tolerance": 2e-2,
                  "pass": bool(err <= 2e-2)}


def copy_write_probe(pk, cache, k_new, v_new, stream, calls=20, pairs_n=192):
    """The two cache-maintenance calls on their own, each timed over `calls`
    back-to-back launches between HIP events: pa_block_copy of `pairs_n`
    (live block, free block) pairs -- the copy-on-write count of the
    prefix-sharing workload -- and pa_kv_write of the step's tokens into
    slots of free blocks.  Only free blocks are written, so the live contexts
    are untouched.  Latency-bound at these sizes: no roofline claim."""
    from paged_kv_cache_335_amd.runtime import DeviceEvent
    k, v = cache.k_pool, cache.v_pool
    B = cache.B
    T = k_new.shape[0]
    free = np.asarray(cache.bm.free_list(), dtype=np.int64)
    n_wblk = (T + B - 1) // B
    if len(free) < pairs_n + n_wblk:
        return None
    S = len(cache.rows)
    live = np.unique(cache.tables[:S, 0].cpu().numpy())  # first block of every sequence
    src = np.resize(live, pairs_n)
    pairs = torch.from_numpy(np.stack([src, free[:pairs_n]], 1).astype(np.int32)).to(k.device)
    slots = (free[pairs_n:pairs_n + n_wblk, None] * B + np.arange(B)).reshape(-1)[:T]
    d_slots = torch.from_numpy(slots.astype(np.int64)).to(k.device)
    block_bytes = k[0].numel() * k.element_size() + v[0].numel() * v.element_size()
    row_bytes = block_bytes // B  # one token's K and V rows, every kv head, in the pool
    res = {}
    for name, fn, moved in (
            ("block_copy", lambda: pk.pa_block_copy(k, v, pairs, stream=stream),
             2 * pairs_n * block_bytes),
            ("kv_write", lambda: pk.pa_kv_write(k, v, k_new, v_new, d_slots, stream=stream),
             T * row_bytes + (k_new.numel() + v_new.numel()) * k_new.element_size())):
        fn()
        a, b = DeviceEvent(timing=True), DeviceEvent(timing=True)
        a.record(stream)
        for _ in range(calls):
            fn()
        b.record(stream)
        b.synchronize()
        us = a.elapsed_ms(b) * 1e3 / calls
        res[name] = {"us": round(us, 2), "bytes_read_and_written": int(moved),
                     "GBps": round(moved / (us * 1e-6) / 1e9, 1)}
    res["block_copy"]["pairs"] = pairs_n
    res["kv_write"]["tokens"] = int(T)
    log(f"block copy of {pairs_n} pairs {res['block_copy']['us']} us; "
        f"slot write of {T} tokens {res['kv_write']['us']} us")
    return res


def swap_probe(pk, cache, n, stream):
    """Swap n resident blocks (K and V, every kv head) out to pinned host
    memory and back into the same device blocks, each direction one
    pa_block_swap launch timed with HIP events; the pools end unchanged."""
    from paged_kv_cache_335_amd.runtime import DeviceEvent
    k, v = cache.k_pool, cache.v_pool
    n = min(n, k.shape[0])
    hk, hv = pk.alloc_host_pools(n, k, v)
    rng = np.random.default_rng(1)
    dev = torch.from_numpy(rng.permutation(k.shape[0])[:n].astype(np.int32))
    host = torch.arange(n, dtype=torch.int32)
    out_pairs = torch.stack([dev, host], 1).contiguous().to(k.device)
    in_pairs = torch.stack([host, dev], 1).contiguous().to(k.device)
    block_bytes = (k[0].numel() * k.element_size() + v[0].numel() * v.element_size())
    res = {}
    for name, pairs, direction in (("out", out_pairs, pk.PA_SWAP_OUT),
                                   ("in", in_pairs, pk.PA_SWAP_IN)):
        best = None
        for _ in range(3):
            a, b = DeviceEvent(timing=True), DeviceEvent(timing=True)
            a.record(stream)
            pk.pa_block_swap(k, v, hk, hv, pairs, direction, stream=stream)
            b.record(stream)
            b.synchronize()
            ms = a.elapsed_ms(b)
            best = ms if best is None else min(best, ms)
        res[name] = {"us": round(best * 1e3, 1),
                     "GBps": round(n * block_bytes / (best * 1e-3) / 1e9, 2)}
    log(f"block swap of {n} blocks ({n * block_bytes / 2**20:.0f} MiB): out "
        f"{res['out']['GBps']} GB/s, in {res['in']['GBps']} GB/s")
    return {"blocks": n, "bytes": int(n * block_bytes), **res}


def cpu_baseline(cache, q, out, lens, S, Hq, d, kv_per_token, seconds):
    """Time the CPU oracle (as it stands) on the last timed step's batch: every
    (sequence, query head) output, repeated until about `seconds` of CPU work
    (a sequence subset when one pass alone would exceed it).  Also compares its
    outputs with the GPU's."""
    import oracle
    from workloads.gen import to_numpy_storage
    log("cpu baseline: copying the pool to the host")
    k = to_numpy_storage(cache.k_pool)
    v = to_numpy_storage(cache.v_pool)
    qn = to_numpy_storage(q)
    tables = cache.tables[:S].cpu().numpy()
    lens = lens.astype(np.int32)
    threads = oracle.max_threads()
    seqs = list(range(S))
    pairs = np.array([[s, h] for s in seqs for h in range(Hq)], np.int32)
    t = time.perf_counter()
    ref = oracle.decode_pairs(k, v, qn, tables, lens, d ** -0.5, pairs)
    one = time.perf_counter() - t
    if one > seconds:
        # one pass is over budget: the longest prefix of a fixed permutation
        # that fits, timed again
        order = np.random.default_rng(0).permutation(S)
        per_token = one / max(1, int(lens.sum()))
        chosen, tok = [], 0
        for s in order:
            if chosen and (tok + lens[s]) * per_token > seconds:
                break
            chosen.append(int(s))
            tok += int(lens[s])
        seqs = chosen
        pairs = np.array([[s, h] for s in seqs for h in range(Hq)], np.int32)
    tok = int(lens[seqs].sum())
    reps, elapsed = 0, 0.0
    while reps == 0 or (elapsed < seconds and reps < 200):
        t = time.perf_counter()
        ref = oracle.decode_pairs(k, v, qn, tables, lens, d ** -0.5, pairs)
        elapsed += time.perf_counter() - t
        reps += 1
    dt = elapsed / reps
    sample_bytes = tok * kv_per_token
    got = out.float().cpu().numpy().astype(np.float64)[pairs[:, 0], pairs[:, 1]]
    err = float(np.abs(got - ref).max())
    log(f"cpu baseline: {len(seqs)} sequences ({tok} tokens) x {reps} passes on {threads} "
        f"threads, {dt:.3f} s per pass, {sample_bytes / dt / 1e9:.3f} GB/s; sampled parity "
        f"max|err| {err:.3e}")
    base = {"value": round(sample_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{len(seqs)} of {S} sequences of the last timed step's batch ({tok} "
                      f"tokens), all {Hq} query heads, {reps} passes ({elapsed:.1f} s); fp64 C "
                      f"oracle, OpenMP over (sequence, head)",
            "seconds_per_pass": round(dt, 4), "tokens_per_s": round(len(seqs) / dt, 3)}
    return base, {"pairs": int(len(pairs)), "max_abs_err": err, "tolerance": 2e-2,
                  "pass": bool(err <= 2e-2)}


if __name__ == "__main__":
    main()
