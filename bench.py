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
private append).  The decode reads each prompt's shared blocks once for its
samples (prefix groups; --no-share reads them per sample).  `value` counts
every sequence's context (logical bytes); the roofline uses the distinct
token slots read (a shared prefix once).

One step = the whole hot path for one batch: the host block manager appends
one token to every sequence (slots, new blocks, copy-on-write decisions),
then one launch (pa_decode_step) stores the 256 new tokens, grows the block
tables and lengths on the device, and runs paged decode attention over
every context; the host's only input to it is each token's block id, read
by the kernel from pinned memory.  (--two-call: a packed host-to-device
metadata copy, pa_kv_append, then pa_decode; the 8-bit cache always takes
this path.)

Prints one JSON line.  `value` is KV bytes read per step / step time (GB/s);
`roofline` reports the decode call (decode and reduce kernels) against the
8 TB/s HBM peak, timed per iteration with HIP events on its stream with the
caches flushed before each iteration (a 512 MiB write outside the events),
median of the iterations (minimum reported beside it), and beside it the
read ceiling a streaming-read probe measures on this GPU.  `cpu_baseline`
times the CPU oracle on a bounded sample of the same batch.  The default
run adds short legs for the other workloads under `legs`.
"""
import argparse
import gc
import hashlib
import json
import math
import os
import subprocess
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention: KV bytes read GB/s (% HBM peak) + decode tokens/s"
HBM_PEAK_GBPS = 8000.0
FLUSH_BYTES = 512 * 1024 * 1024


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "decode_hbm_traffic.md")
DECODE_SOURCES = ("paged_kv_cache_335_amd/csrc/pa_decode.hip",
                  "paged_kv_cache_335_amd/csrc/pa_device.h",
                  "paged_kv_cache_335_amd/csrc/pa_internal.h")


def decode_source_hash():
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, algorithmic_bytes):
    """HBM bytes per decode launch: the traffic / algorithmic-bytes ratio that
    the committed counter summary records for this workload (FETCH_SIZE and
    WRITE_SIZE passes, scaled by a plain copy's counters), applied to this
    run's algorithmic bytes; None when the decode sources changed since the
    counters were taken or the summary has no entry for the workload."""
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    src = None
    ratios = {}
    for ln in text.splitlines():
        if ln.startswith("decode_source_sha256: "):
            src = ln.split(": ", 1)[1].strip()
        elif ln.startswith("traffic_ratio "):
            key, val = ln[len("traffic_ratio "):].split(": ", 1)
            ratios[key.strip()] = float(val)
    if src != decode_source_hash() or workload not in ratios:
        return None
    return {"bytes_per_launch": int(round(ratios[workload] * algorithmic_bytes)),
            "ratio_to_algorithmic": ratios[workload],
            "source": os.path.relpath(TRAFFIC_PROFILE, ROOT)}


def cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
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
    ap.add_argument("--extend-prefix", type=int, default=0,
                    help="extend: every sequence's cached prefix (0: the workload's lengths)")
    ap.add_argument("--chunk", type=int, default=256, help="new tokens per sequence per step")
    ap.add_argument("--no-share", action="store_true",
                    help="prefix-sharing configs: read shared blocks once per sequence, not "
                         "once per prefix group")
    ap.add_argument("--two-call", action="store_true",
                    help="run each step as pa_kv_append then pa_decode instead of the fused "
                         "pa_decode_step")
    ap.add_argument("--kv", default="bf16", choices=["bf16", "fp8"],
                    help="cache storage: bf16, or 8-bit E4M3 codes + per-token scales")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-iters", type=int, default=50,
                    help="decode iterations timed one by one with the caches flushed before each")
    ap.add_argument("--no-legs", action="store_true",
                    help="skip the short legs of the other workloads")
    ap.add_argument("--leg-steps", type=int, default=10)
    ap.add_argument("--leg-only", action="store_true",
                    help="run one workload as a leg (short form) and print its JSON; the "
                         "default run starts one such process per leg")
    ap.add_argument("--no-read-probe", action="store_true")
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

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(dev)
    torch.cuda.set_stream(stream)

    if args.mode == "extend":
        return bench_extend(args, pk, DeviceEvent, PagedKVCache, CONFIGS, draw_lengths)
    if args.leg_only:
        leg = run_decode(args, args.config, args.kv, args.block_size, args.steps, args.warmup,
                         max(1, args.cold_iters), stream, full=False)
        print(json.dumps(leg), flush=True)
        return

    res = run_decode(args, args.config, args.kv, args.block_size, args.steps, args.warmup,
                     max(1, args.cold_iters), stream, full=True)
    result = res.pop("result")
    if not args.no_read_probe:
        result["read_ceiling"] = read_probe(pk, stream)
        result["roofline"]["measured_read_ceiling_GBps"] = \
            result["read_ceiling"]["random_16KiB_chunks"]["GBps"]
    if not args.no_legs and args.config == "llama3_8b_gqa" and args.kv == "bf16" \
            and args.block_size == 16 and args.partition == 0:
        # Each leg runs in a process of its own, as a standalone run of that
        # workload would: run in this process after the others, the 8-bit
        # and block-size legs read 2-6% slower than standalone runs on the
        # same box (the allocator's history, not the kernels).
        torch.cuda.synchronize()
        gc.collect()
        torch.cuda.empty_cache()
        legs = {}
        for name, key, kv, B in (("llama2_7b_mha", "llama2_7b_mha", "bf16", 16),
                                 ("prefix_sharing", "prefix_sharing", "bf16", 16),
                                 ("prefix_sharing_cow", "prefix_sharing_cow", "bf16", 16),
                                 ("long_context_128k", "long_context_128k", "bf16", 16),
                                 ("llama3_8b_gqa_fp8", "llama3_8b_gqa", "fp8", 16),
                                 ("llama3_8b_gqa_block32", "llama3_8b_gqa", "bf16", 32),
                                 ("llama3_8b_gqa_block8", "llama3_8b_gqa", "bf16", 8)):
            legs[name] = run_leg(args, key, kv, B)
        result["legs"] = legs
    print(json.dumps(result), flush=True)


def run_leg(args, key, kv, block_size):
    """One leg in a child process (this script with --leg-only); its JSON, or
    an error record if the child failed."""
    cmd = [sys.executable, "-u", os.path.abspath(__file__), "--leg-only", "--config", key,
           "--kv", kv, "--block-size", str(block_size), "--steps", str(args.leg_steps),
           "--warmup", "3", "--cold-iters", str(max(5, args.cold_iters // 2))]
    if args.two_call:
        cmd.append("--two-call")
    try:
        out = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=None, text=True, timeout=600,
                             cwd=ROOT)
    except subprocess.TimeoutExpired:
        return {"error": "timed out"}
    lines = [ln for ln in out.stdout.splitlines() if ln.startswith("{")]
    if out.returncode != 0 or not lines:
        return {"error": f"exit status {out.returncode}"}
    return json.loads(lines[-1])


def run_decode(args, key, kv, block_size, K, W, cold_iters, stream, full):
    """One workload: build and fill the cache through the slot write, time K
    whole steps after W warm-up steps, then the decode call alone (warm back
    to back, and cold: caches flushed before each iteration).  full=True
    adds the cache-op and swap probes and the CPU oracle baseline and
    returns the whole JSON line under "result"; otherwise a compact dict."""
    import paged_kv_cache_335_amd as pk
    from paged_kv_cache_335_amd.runtime import DeviceEvent, PagedKVCache
    from workloads import CONFIGS, draw_lengths
    from workloads.gen import unique_blocks

    cfg = CONFIGS[key]
    if block_size != cfg.block_size:
        cfg = cfg.scaled(block_size=block_size)
    dev = torch.device("cuda:0")
    S, Hq, Hkv, d, B = cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
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
    fp8 = kv == "fp8"
    share = bool(shared) and not args.no_share
    tag = f"{cfg.key}{' fp8' if fp8 else ''}{'' if B == 16 else f' B={B}'}"
    log(f"{tag}: S={S} Hq={Hq} Hkv={Hkv} d={d} sum L={int(lens0.sum())} "
        f"pool={num_blocks} blocks width={width}{' (prefix groups)' if share else ''}")

    cache = PagedKVCache(num_blocks, Hkv, d, S, width, block_size=B, shuffle_seed=cfg.seed,
                         dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev,
                         share_prefixes=share, max_group=max(1, 16 // (Hq // Hkv)))
    g = torch.Generator(device=dev)
    g.manual_seed(cfg.seed)
    if shared:
        # each prompt's shared tokens once, then its forks (so a prompt's
        # samples take adjacent table rows)
        seq_list = []
        for _ in range(cfg.prompts):
            s0 = cache.add_sequence()
            kn = torch.randn((shared, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
            vn = torch.randn((shared, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
            cache.append(np.array([s0], np.int32), np.array([shared], np.int32), kn, vn,
                         stream=stream)
            seq_list += [s0] + [cache.fork(s0, stream=stream) for _ in range(cfg.samples - 1)]
        seqs = np.array(seq_list, dtype=np.int32)
    else:
        seqs = np.array([cache.add_sequence() for _ in range(S)], dtype=np.int32)

    # prefill: every context token but the one each first step appends (past
    # the shared prefix, which is already in place)
    pre = (lens0 - 1 - shared).astype(np.int32)
    chunk = 16384
    start = 0
    while start < S:
        # batches of whole sequences, about `chunk` tokens each
        tot, end = 0, start
        while end < S and (tot == 0 or tot + pre[end] <= chunk):
            tot += int(pre[end])
            end += 1
        kn = torch.randn((tot, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
        vn = torch.randn((tot, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
        cache.append(seqs[start:end], pre[start:end], kn, vn, stream=stream)
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

    fused = not args.two_call

    def step(i):
        if fused:   # one launch: slot write, table growth and decode (pa_decode_step)
            cache.step(qs[i], kns[i], vns[i], out=out, partition_tokens=args.partition,
                       stream=stream)
        else:       # pa_kv_append, then pa_decode
            cache.append(seqs, ones, kns[i], vns[i], stream=stream)
            cache.decode(qs[i], out=out, partition_tokens=args.partition, stream=stream)

    # Python's cyclic garbage collector: a full collection takes tens of
    # milliseconds in this process and, when one fell inside the timed steps,
    # left the GPU idle for a few steps' worth of time.  Collect before the
    # warm-up (whose steps then also warm the host path) and keep it off
    # until the timed steps and the decode timings have run.
    gc.collect()
    gc.disable()
    for i in range(W):
        step(i)
        step_bytes.append(int(cache.host_lens[:S].sum()) * kv_per_token)
        step_unique.append(unique_tokens(cache.host_lens[:S]) * kv_per_token)
    torch.cuda.synchronize()
    # the timed steps carry no events: recording one leaves the GPU idle for
    # a few microseconds before the next kernel, which is instrumentation,
    # not part of the path
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
    kv_avg = float(np.mean(step_bytes[W:]))
    value = kv_avg / (ms_step * 1e-3) / 1e9
    last_bytes, last_unique = step_bytes[-1], step_unique[-1]

    def decode_call():
        cache.decode(qs[-1], out=out, partition_tokens=args.partition, stream=stream)

    # warm: K decode calls back to back over the last step's batch, between
    # two fence-free HIP events on the decode stream
    ea, eb = DeviceEvent(timing=True), DeviceEvent(timing=True)
    ea.record(stream)
    for _ in range(K):
        decode_call()
    eb.record(stream)
    eb.synchronize()
    warm_us = ea.elapsed_ms(eb) / K * 1e3

    # cold: each iteration timed on its own, the caches (L2 and the last-level
    # cache) flushed before it by a 512 MiB write outside the events
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    evs = [(DeviceEvent(timing=True), DeviceEvent(timing=True)) for _ in range(cold_iters)]
    for i in range(5 + cold_iters):
        flush.fill_(float(i))
        if i >= 5:
            evs[i - 5][0].record(stream)
        decode_call()
        if i >= 5:
            evs[i - 5][1].record(stream)
    torch.cuda.synchronize()
    gc.enable()  # off since before the warm-up
    cold_us = np.array([a.elapsed_ms(b) * 1e3 for a, b in evs])
    del flush
    med, mn = float(np.median(cold_us)), float(np.min(cold_us))
    roof_bytes = last_unique  # a shared prefix counts once
    achieved = roof_bytes / (med * 1e-6) / 1e9
    log(f"{tag}: step {ms_step:.3f} ms ({value:.0f} GB/s); decode warm {warm_us:.1f} us, "
        f"cold median {med:.1f} us (min {mn:.1f}) = {achieved:.0f} GB/s "
        f"({achieved / HBM_PEAK_GBPS:.3f} of peak); host enqueue {host_ms:.3f} ms/step")

    workload = f"{cfg.key}/{kv}/B{B}" + ("/shared" if share else "") + (
        f"/P{args.partition}" if args.partition else "")
    traffic = measured_traffic(workload, roof_bytes)
    total_blocks = int(((cache.host_lens[:S].astype(np.int64) + B - 1) // B).sum())
    piece = pk.pa_decode_piece_tokens(cache.k_pool, cache.v_pool, S, Hq, width, total_blocks,
                                      args.partition)
    lens_now = cache.host_lens[:S].copy()
    pieces = int(np.sum(-(-lens_now.astype(np.int64) // piece))) if piece else None
    decode = {"us_warm": round(warm_us, 2), "us_cold_median": round(med, 2),
              "us_cold_min": round(mn, 2), "cold_iters": int(cold_iters),
              "kv_bytes": int(last_bytes), "kv_bytes_unique": int(roof_bytes),
              "GBps_cold_median": round(achieved, 1),
              "GBps_cold_best": round(roof_bytes / (mn * 1e-6) / 1e9, 1),
              "GBps_warm": round(roof_bytes / (warm_us * 1e-6) / 1e9, 1),
              "GBps_logical_cold_median": round(last_bytes / (med * 1e-6) / 1e9, 1),
              "tokens_per_s": round(S / (med * 1e-6), 1),
              "piece_tokens": piece, "pieces_about": pieces,
              "prefix_groups": int(cache.num_groups) if share else None}
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic["bytes_per_launch"] if traffic else None,
                "timing": f"decode call (decode + reduce kernels), median of {cold_iters} "
                          "iterations, each between its own HIP events, caches flushed before "
                          "each; bytes = distinct K/V token slots read"}
    if traffic:
        roofline["traffic_ratio"] = traffic["ratio_to_algorithmic"]
        roofline["traffic_source"] = traffic["source"]

    if not full:
        res = {"workload": f"{cfg.key}: {cfg.description}" + (
                   "; 8-bit cache" if fp8 else "") + (f"; {B}-token blocks" if B != 16 else ""),
               "step": "pa_decode_step (one launch)" if fused else "pa_kv_append + pa_decode",
               "steps": K, "warmup": W, "ms_per_step": round(ms_step, 5),
               "step_GBps": round(value, 1), "decode": decode, "roofline": roofline}
        del cache, qs, kns, vns, out
        gc.collect()
        torch.cuda.empty_cache()
        return res

    # the last step's output again, for the sampled parity check below
    decode_call()
    torch.cuda.synchronize()
    copy_write = copy_write_probe(pk, cache, kns[-1], vns[-1], stream)
    swap = swap_probe(pk, cache, args.swap_blocks, stream) if args.swap_blocks > 0 else None
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * 1024 * 1024 // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: {args.copy_probe_mib} MiB read + {args.copy_probe_mib} MiB written")
        del src, dst

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
            "kv_storage": kv,
            "num_seqs": S, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": d,
            "block_size": B, "pool_blocks": num_blocks, "partition_tokens": P,
            "step": "pa_decode_step (one launch)" if fused else "pa_kv_append + pa_decode",
            "mean_context_tokens": round(float(lens_now.mean()), 1),
            "kv_bytes_per_step": int(kv_avg),
            "kv_bytes_unique_per_step": int(np.mean(step_unique[W:])),
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "tokens_per_s": round(S / (ms_step * 1e-3), 1),
        "host_enqueue_ms_per_step": round(host_ms, 4),
        "decode": decode,
        "roofline": roofline,
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
    del cache, qs, kns, vns, out
    gc.collect()
    torch.cuda.empty_cache()
    return {"result": result}


def read_probe(pk, stream, total_bytes=2 << 30, reps=3):
    """The read ceiling of this GPU: a 2 GiB buffer read once per pass with
    16-byte non-temporal loads (pa_probe_read), as a contiguous stream (1 MiB
    chunks in order) and as gathers of 16 KiB and 4 KiB chunks in random
    order (the regions a decode workgroup and a wave read per block).  Each
    pattern is tried at 1, 2, 4 and 8 workgroups per CU with 2 and 8 loads
    in flight per thread; the best pass (each between its own HIP events)
    is the ceiling."""
    from paged_kv_cache_335_amd.runtime import DeviceEvent
    dev = torch.device("cuda:0")
    buf = torch.empty(total_bytes, dtype=torch.uint8, device=dev)
    buf.fill_(7)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(int(pk.lib().pa_probe_sink_bytes(cus * 8)), dtype=torch.uint8, device=dev)
    rng = np.random.default_rng(0)
    res = {}
    for name, chunk, shuffled in (("contiguous", 1 << 20, False),
                                  ("random_16KiB_chunks", 16 << 10, True),
                                  ("random_4KiB_chunks", 4 << 10, True)):
        n = total_bytes // chunk
        order = rng.permutation(n) if shuffled else np.arange(n)
        d_order = torch.from_numpy(order.astype(np.int32)).to(dev)
        best = None
        for per_cu in (1, 2, 4, 8):
            for lif in (2, 8):
                wgs = cus * per_cu
                pk.pa_probe_read(buf, d_order, chunk, wgs, lif, sink=sink, stream=stream)
                for _ in range(reps):
                    a, b = DeviceEvent(timing=True), DeviceEvent(timing=True)
                    a.record(stream)
                    pk.pa_probe_read(buf, d_order, chunk, wgs, lif, sink=sink, stream=stream)
                    b.record(stream)
                    b.synchronize()
                    ms = a.elapsed_ms(b)
                    if best is None or ms < best[0]:
                        best = (ms, per_cu, lif)
        gbps = total_bytes / (best[0] * 1e-3) / 1e9
        res[name] = {"chunk_bytes": chunk, "GBps": round(gbps, 1),
                     "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
                     "workgroups_per_cu": best[1], "loads_in_flight": best[2]}
    log("read ceiling: " + ", ".join(f"{k} {v['GBps']:.0f} GB/s" for k, v in res.items()))
    del buf, sink
    torch.cuda.empty_cache()
    res["method"] = ("pa_probe_read over a 2 GiB buffer, 16-byte non-temporal loads, 256 "
                     "threads per workgroup; best pass over 1-8 workgroups per CU and 2 or 8 "
                     "loads in flight per thread")
    return res


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
    if args.extend_prefix > 0:
        lens0 = np.full(S, args.extend_prefix, np.int64)
    else:
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
    # the split (and its workspace) depends only on the batch shape and table width
    ws_bytes = pk.pa_extend_workspace_bytes(cache.k_pool, cache.v_pool, T, S, Hq, width)
    workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    log(f"extend workspace {ws_bytes} bytes")

    last = {}

    def step(i):
        cache.append(seqs, ns, kns[i], vns[i], stream=stream)
        tables, lens = cache.bm.export(seqs, width, pad_block=0)
        d_tables = torch.from_numpy(tables).to(dev, non_blocking=False)
        d_lens = torch.from_numpy(lens).to(dev, non_blocking=False)
        last.update(q=qs[i], tables=d_tables, lens=d_lens)
        ev[i][0].record(stream)
        pk.pa_extend(qs[i], cache.k_pool, cache.v_pool, q_start, d_tables, d_lens, scale,
                     out=out, workspace=workspace, stream=stream)
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
    # per-step events bracket each launch, and with the device idle after the
    # step's host work they also take in the host's launch latency; the
    # kernel's own rate comes from K launches back to back over the last
    # step's batch, between two events on the extend stream
    ext_ms = [ev[i][0].elapsed_ms(ev[i][1]) for i in range(W, steps)]
    ea, eb = DeviceEvent(timing=True), DeviceEvent(timing=True)
    ea.record(stream)
    for _ in range(K):
        pk.pa_extend(last["q"], cache.k_pool, cache.v_pool, q_start, last["tables"], last["lens"],
                     scale, out=out, workspace=workspace, stream=stream)
    eb.record(stream)
    torch.cuda.synchronize()
    ext_avg = ea.elapsed_ms(eb) / K
    fl = float(flops[-1])
    tflops = fl / (ext_avg * 1e-3) / 1e12
    log(f"extend step {ms_step:.3f} ms; attention {ext_avg * 1e3:.1f} us back to back "
        f"({float(np.mean(ext_ms)) * 1e3:.1f} us per step event), {tflops:.1f} TFLOP/s")
    result = {
        "metric": "paged extend (chunked prefill) attention: TFLOP/s + query tokens/s",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{cfg.key} shape, {S} sequences with cached prefixes, "
                               f"{C}-token chunks", "num_seqs": S, "chunk": C,
                   "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": d, "block_size": B,
                   "mean_context_tokens": round(float(np.mean(lens0)) + (W + K) * C / 2, 1)},
        "extend": {"us_back_to_back": round(ext_avg * 1e3, 2),
                   "us_step_event_mean": round(float(np.mean(ext_ms)) * 1e3, 2),
                   "query_tokens_per_s": round(T / (ext_avg * 1e-3), 1),
                   "kv_GBps_unique": round(float(kv_bytes[-1]) / (ext_avg * 1e-3) / 1e9, 1)},
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
            "kind": "oracle", "cpu_model": cpu_model(),
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
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{len(seqs)} of {S} sequences of the last timed step's batch ({tok} "
                      f"tokens), all {Hq} query heads, {reps} passes ({elapsed:.1f} s); fp64 C "
                      f"oracle, OpenMP over (sequence, head)",
            "seconds_per_pass": round(dt, 4), "tokens_per_s": round(len(seqs) / dt, 3)}
    return base, {"pairs": int(len(pairs)), "max_abs_err": err, "tolerance": 2e-2,
                  "pass": bool(err <= 2e-2)}


if __name__ == "__main__":
    main()
