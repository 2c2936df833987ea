"""Filling large K/V pools on the GPU from a seeded torch generator.

The headline and long-context workloads carry pools of 0.6-2 GB per layer,
too large to draw on the host for every run.  Here each pool is drawn as
N(0, 1) directly in bf16 by torch's device generator, seeded from the same
(workload, stream, layer) key as the host streams.  A checker that needs
the values copies the pool back to the host.
"""
from __future__ import annotations

import torch

from .generate import stream_seed


def device_pool(cfg, num_blocks: int, stream: str, layer: int, device="cuda") -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(stream_seed(cfg.seed, stream, layer))
    shape = (num_blocks, cfg.block_size, cfg.num_kv_heads, cfg.head_dim)
    return torch.randn(shape, generator=g, device=device, dtype=torch.bfloat16)


def device_normal_bf16(seed: int, shape, device="cuda") -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.bfloat16)
