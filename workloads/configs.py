"""The five decode workloads.

Each one is a single decode step: every row's new token (the last of its
n_b context positions) is stored into a paged K/V pool and then attends to
all n_b cached positions; the sampler then draws one id per row.

Shapes follow the workloads named for this library:
  1 tiny      - one layer, four rows, MHA 16/16, head_dim 64
  2 qwen3     - Qwen3-0.6B-shaped: 64 rows, GQA 16/8, 28 layers (the headline)
  3 grok      - Grok-1-shaped static batch: 32 rows padded to 2048, GQA 48/8
  4 clone     - one prompt cloned 16 ways: a shared 1024-token prefix
  5 long      - long-context split-KV stress: 8 rows of 32K-128K tokens
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class DecodeConfig:
    index: int                  # 1-based workload number
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_layers: int
    vocab: int
    logit_std: float            # logits ~ N(0, logit_std), std-dev convention
    temperature: float
    top_p: float
    top_k: int
    # context-length recipe
    ctx_kind: str               # "fixed" | "uniform" | "clone"
    ctx_fixed: tuple = field(default_factory=tuple)
    ctx_lo: int = 0
    ctx_hi: int = 0
    # block-table recipe
    table_kind: str = "perm"    # "perm" | "contiguous" | "clone"
    pool_blocks: int = 0        # 0: derived (sum of blocks used + 5% spare)
    clone_prefix_blocks: int = 0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def seed(self) -> int:
        # base seed 42 (the Grok-1 runner's default request seed), one
        # independent family of streams per workload
        return 42 + 1000 * self.index


CONFIGS = [
    DecodeConfig(1, "tiny", batch=4, num_q_heads=16, num_kv_heads=16, head_dim=64,
                 block_size=256, num_layers=1, vocab=32768, logit_std=2.0,
                 temperature=0.7, top_p=1.0, top_k=0,
                 ctx_kind="fixed", ctx_fixed=(17, 256, 299, 513),
                 table_kind="perm", pool_blocks=16),
    DecodeConfig(2, "qwen3", batch=64, num_q_heads=16, num_kv_heads=8, head_dim=128,
                 block_size=256, num_layers=28, vocab=151936, logit_std=3.0,
                 temperature=0.8, top_p=0.95, top_k=0,
                 ctx_kind="uniform", ctx_lo=128, ctx_hi=4096,
                 table_kind="perm", pool_blocks=0),
    DecodeConfig(3, "grok", batch=32, num_q_heads=48, num_kv_heads=8, head_dim=128,
                 block_size=256, num_layers=1, vocab=131072, logit_std=4.0,
                 temperature=0.01, top_p=1.0, top_k=0,
                 ctx_kind="fixed", ctx_fixed=(2048,) * 32,
                 table_kind="contiguous", pool_blocks=256),
    DecodeConfig(4, "clone", batch=16, num_q_heads=10, num_kv_heads=10, head_dim=128,
                 block_size=256, num_layers=1, vocab=65536, logit_std=3.0,
                 temperature=1.0, top_p=1.0, top_k=50,
                 ctx_kind="clone", ctx_lo=0, ctx_hi=256,
                 table_kind="clone", pool_blocks=0, clone_prefix_blocks=4),
    DecodeConfig(5, "long", batch=8, num_q_heads=64, num_kv_heads=8, head_dim=128,
                 block_size=256, num_layers=1, vocab=151936, logit_std=3.0,
                 temperature=1.0, top_p=0.9, top_k=0,
                 ctx_kind="uniform", ctx_lo=32768, ctx_hi=131072,
                 table_kind="perm", pool_blocks=4096),
]


def config_by_name(name_or_index) -> DecodeConfig:
    for c in CONFIGS:
        if c.name == name_or_index or str(c.index) == str(name_or_index):
            return c
    raise KeyError(f"unknown workload {name_or_index!r}")
