"""The five synthetic decode workloads (plus a copy-on-write variant).

Each entry fixes the shape of one decode batch: sequence count, query and KV
head counts, head dim, storage dtype, block size 16, the length mix, the pool
size and the seed.  Sizes are given in full; tests scale some of them down
with ``Config.scaled`` so the CPU oracle finishes in seconds.
"""
from dataclasses import dataclass, replace
import math


@dataclass(frozen=True)
class Config:
    key: str
    description: str
    seed: int
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str                 # pool storage: "f32", "bf16" or "fp8" (E4M3 + scales)
    block_size: int
    lengths: tuple             # see gen.draw_lengths
    pool: tuple                # ("fixed", n_blocks) or ("plus", fraction)
    table_width: int           # max_blocks_per_seq of the block table
    partition_tokens: int = 0  # 0: the library picks
    kv_write_tokens: int = 0   # tokens written per decode step
    prompts: int = 0           # prefix-sharing configs: number of prompts
    samples: int = 0           # prefix-sharing configs: samples per prompt

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def scaled(self, **kw) -> "Config":
        return replace(self, **kw)


CONFIGS = {
    "tiny_f32": Config(
        key="tiny_f32", description="tiny fp32: 4 seqs, L~U[1,64], 1 head, d=64, 32-block pool",
        seed=1, num_seqs=4, num_q_heads=1, num_kv_heads=1, head_dim=64, dtype="f32",
        block_size=16, lengths=("uniform", 1, 64), pool=("fixed", 32), table_width=8),
    "llama2_7b_mha": Config(
        key="llama2_7b_mha", description="Llama-2-7B-shape MHA 32/32, d=128, bf16, batch 64, L~U[128,2048]",
        seed=2, num_seqs=64, num_q_heads=32, num_kv_heads=32, head_dim=128, dtype="bf16",
        block_size=16, lengths=("uniform", 128, 2048), pool=("fixed", 16384),
        table_width=128),
    "llama3_8b_gqa": Config(
        key="llama3_8b_gqa",
        description="Llama-3-8B-shape GQA 32/8, d=128, bf16, batch 256, L~lognormal(median 1024,"
                    " sigma 1) clipped to [16,8192], pool = blocks + 10%, 256-token slot write",
        seed=3, num_seqs=256, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
        block_size=16, lengths=("lognormal", 1024, 1.0, 16, 8192), pool=("plus", 0.10),
        table_width=512, kv_write_tokens=256),
    "prefix_sharing": Config(
        key="prefix_sharing",
        description="prefix sharing: 64 prompts x 4 samples, 1024 shared tokens, private"
                    " U[1,256], GQA 32/8, d=128, bf16",
        seed=4, num_seqs=256, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
        block_size=16, lengths=("shared", 1024, 1, 256), pool=("plus", 0.10),
        table_width=80, prompts=64, samples=4),
    "prefix_sharing_cow": Config(
        key="prefix_sharing_cow",
        description="prefix sharing with a partly filled shared tail: 1032 shared tokens"
                    " (64 full blocks + 8), so each fork but the last copies the tail",
        seed=4, num_seqs=256, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
        block_size=16, lengths=("shared", 1032, 1, 256), pool=("plus", 0.10),
        table_width=81, prompts=64, samples=4),
    "long_context_128k": Config(
        key="long_context_128k",
        description="long context: batch 4 x 131072 tokens, GQA 32/8, d=128, bf16, 32768"
                    " scattered blocks, split over 512-token partitions",
        seed=5, num_seqs=4, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
        block_size=16, lengths=("fixed", 131072), pool=("fixed", 32768), table_width=8192,
        partition_tokens=512),
}


def get_config(key: str) -> Config:
    return CONFIGS[key]
