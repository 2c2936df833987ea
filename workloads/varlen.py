"""Seeded inputs for varlen multi-query (chunked prefill) attention.

A workload is a batch of sequences, each with a cached prefix already in
the paged cache and a chunk of new tokens whose K/V are stored before the
attention runs.  Values follow the decode workloads: N(0, 1) rounded to
bf16 for q, new K/V and every pool byte; fragmented block tables from a
seeded permutation.  No attention arithmetic lives here.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .generate import normal_bf16


@dataclass(frozen=True)
class VarlenWorkload:
    name: str
    lens_cached: tuple       # tokens already in the cache, per sequence
    lens_new: tuple          # new tokens of this chunk, per sequence
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_layers: int
    seed: int

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


# Qwen3-0.6B-shaped chunked prefill: 4 sequences, 512 new tokens each, after
# cached prefixes of 0 / 256 / 1024 / 1536 tokens (GQA 16/8, D 128, block 256,
# 28 layers); and one long-prefix chunk (4 layers).
VARLEN_WORKLOADS = [
    VarlenWorkload("qwen3_prefill", (0, 256, 1024, 1536), (512, 512, 512, 512), 16, 8, 128, 256,
                   28, 42 + 1000 * 6),
    # one sequence, a 512-token chunk after a 16384-token cached prefix: only
    # 64 (row tile, KV head) pairs, so the causal ranges are split
    VarlenWorkload("qwen3_long_prefix", (16384,), (512,), 16, 8, 128, 256, 4, 42 + 1000 * 7),
]


def varlen_by_name(name: str) -> VarlenWorkload:
    for w in VARLEN_WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)


def _rng(seed: int, stream: int, layer: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, 100 + stream, layer])


def varlen_tables(w: VarlenWorkload):
    """(tables int32 [B, W], cu_seqlens_q [B+1], cu_seqlens_k [B+1], num_blocks)."""
    total = [c + n for c, n in zip(w.lens_cached, w.lens_new)]
    bs = w.block_size
    need = [max(1, (t + bs - 1) // bs) for t in total]
    nb = sum(need) + 2
    perm = _rng(w.seed, 1).permutation(nb).astype(np.int32)
    tables = np.full((len(total), max(need)), -1, np.int32)
    pos = 0
    for b, k in enumerate(need):
        tables[b, :k] = perm[pos:pos + k]
        pos += k
    cu_q = np.concatenate([[0], np.cumsum(w.lens_new)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(total)]).astype(np.int32)
    return tables, cu_q, cu_k, nb


def varlen_layer_inputs(w: VarlenWorkload, layer: int):
    """q uint16 [T, Hq, D] and the new tokens' k, v uint16 [T, Hkv, D]."""
    T = int(sum(w.lens_new))
    q = normal_bf16(_rng(w.seed, 2, layer), (T, w.num_q_heads, w.head_dim))
    k = normal_bf16(_rng(w.seed, 3, layer), (T, w.num_kv_heads, w.head_dim))
    v = normal_bf16(_rng(w.seed, 4, layer), (T, w.num_kv_heads, w.head_dim))
    return q, k, v


def varlen_attended_pairs(w: VarlenWorkload) -> int:
    """(query token, key position) pairs under the causal mask, per head."""
    return int(sum(c * n + n * (n + 1) // 2 for c, n in zip(w.lens_cached, w.lens_new)))
