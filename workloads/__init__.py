"""Seeded synthetic inputs for paged decode attention.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no attention, no slot arithmetic beyond building a valid
table, no copies).  It is the one module both the GPU path's tests and the
oracle consume.

Workload shapes (sequence counts, head counts, head dim, length mixes, pool
sizes) are those of the five synthetic decode configurations this project is
measured on; see ``CONFIGS``.  Values are N(0, 1) in float32 rounded to
bfloat16 (round to nearest even) where the storage is bf16.
"""
from .configs import CONFIGS, Config, get_config  # noqa: F401
from .gen import (  # noqa: F401
    POISON_K,
    POISON_V,
    BlockCopyCase,
    DecodeCase,
    KVWriteCase,
    bf16_bits_to_f32,
    block_copy_case,
    decode_case,
    decode_structure,
    draw_lengths,
    f32_to_bf16_bits,
    kv_write_case,
)
