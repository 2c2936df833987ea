"""Seeded generation of decode-step inputs.

Every tensor comes from its own named stream so that, e.g., asking for more
layers never changes the logits.  Streams are numpy PCG64 generators keyed
by (workload seed, stream id, layer).  Large K/V pools can instead be filled
on the GPU from a torch generator seeded by the same key (see ``device.py``);
whoever checks them then copies the filled pools back to the host.

Values:
  * K/V pools, q, k_new, v_new: N(0, 1) rounded to bf16 (round to nearest
    even), stored as uint16 bit patterns.  Every pool block, used or not, is
    filled, so a wrong gather reads visibly different data.
  * logits: N(0, logit_std) in fp32 (std-dev convention).
  * gumbel: standard Gumbel(0, 1) noise, drawn in fp64 and rounded to fp32.
    The noise is an input of the sampler, so the device never draws it.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import DecodeConfig

_STREAMS = {
    "lengths": 1, "perm": 2, "kpool": 3, "vpool": 4, "q": 5,
    "knew": 6, "vnew": 7, "logits": 8, "gumbel": 9, "tails": 10,
}


def stream_seed(cfg_seed: int, stream: str, layer: int = 0) -> int:
    """A 63-bit seed for one named stream (used to seed torch generators)."""
    ss = np.random.SeedSequence([cfg_seed, _STREAMS[stream], layer])
    return int(ss.generate_state(1, dtype=np.uint64)[0]) & ((1 << 63) - 1)


def _rng(cfg_seed: int, stream: str, layer: int = 0) -> np.random.Generator:
    return np.random.default_rng([cfg_seed, _STREAMS[stream], layer])


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return bf16_bits_from_f32(rng.standard_normal(size=shape, dtype=np.float32))


def context_lengths(cfg: DecodeConfig) -> np.ndarray:
    """n_b per row, counting the new token (positions 0..n_b-1)."""
    if cfg.ctx_kind == "fixed":
        n = np.asarray(cfg.ctx_fixed, dtype=np.int64)
        assert n.shape == (cfg.batch,)
    elif cfg.ctx_kind == "uniform":
        n = _rng(cfg.seed, "lengths").integers(cfg.ctx_lo, cfg.ctx_hi, size=cfg.batch,
                                               endpoint=True)
    elif cfg.ctx_kind == "clone":
        # a shared prefix of clone_prefix_blocks full blocks, then t_b cached
        # divergent tokens, then the new token at position prefix + t_b
        tails = _rng(cfg.seed, "tails").integers(cfg.ctx_lo, cfg.ctx_hi, size=cfg.batch,
                                                 endpoint=True)
        n = cfg.clone_prefix_blocks * cfg.block_size + tails + 1
    else:
        raise ValueError(cfg.ctx_kind)
    return n.astype(np.int32)


def block_tables(cfg: DecodeConfig, n: np.ndarray):
    """Physical block ids per row, int32 [B, max_blocks]; unused entries -1.

    Returns (tables, num_blocks)."""
    bs = cfg.block_size
    need = [(int(x) + bs - 1) // bs for x in n]
    width = max(1, max(need))
    tables = np.full((cfg.batch, width), -1, dtype=np.int32)
    if cfg.table_kind == "perm":
        total = sum(need)
        nb = cfg.pool_blocks if cfg.pool_blocks else int(math.ceil(total * 1.05))
        assert nb >= total, "pool too small for the drawn lengths"
        perm = _rng(cfg.seed, "perm").permutation(nb).astype(np.int32)
        pos = 0
        for b in range(cfg.batch):
            tables[b, :need[b]] = perm[pos:pos + need[b]]
            pos += need[b]
    elif cfg.table_kind == "contiguous":
        nb = cfg.pool_blocks
        for b in range(cfg.batch):
            tables[b, :need[b]] = np.arange(b * width, b * width + need[b], dtype=np.int32)
        assert nb >= cfg.batch * width
    elif cfg.table_kind == "clone":
        pre = cfg.clone_prefix_blocks
        private = [x - pre for x in need]
        assert min(private) >= 1
        nb = pre + sum(private)
        perm = _rng(cfg.seed, "perm").permutation(nb).astype(np.int32)
        shared = perm[:pre]
        pos = pre
        for b in range(cfg.batch):
            tables[b, :pre] = shared
            tables[b, pre:need[b]] = perm[pos:pos + private[b]]
            pos += private[b]
    else:
        raise ValueError(cfg.table_kind)
    return tables, int(nb)


@dataclass
class HostInputs:
    cfg: DecodeConfig
    context_lens: np.ndarray          # int32 [B]
    block_tables: np.ndarray          # int32 [B, W]
    num_blocks: int
    layers: list                      # layer indices generated
    q: list                           # per layer uint16 [B, Hq, D]
    k_new: list                       # per layer uint16 [B, Hkv, D]
    v_new: list
    k_pool: Optional[list]            # per layer uint16 [NB, bs, Hkv, D] or None
    v_pool: Optional[list]
    logits: Optional[np.ndarray]      # fp32 [B, V]
    gumbel: Optional[np.ndarray]      # fp32 [B, V]
    temperature: np.ndarray           # fp32 [B]
    top_p: np.ndarray                 # fp32 [B]
    top_k: np.ndarray                 # int32 [B]


def sampling_params(cfg: DecodeConfig):
    B = cfg.batch
    return (np.full(B, cfg.temperature, np.float32), np.full(B, cfg.top_p, np.float32),
            np.full(B, cfg.top_k, np.int32))


def host_inputs(cfg: DecodeConfig, layers=(0,), pools: bool = True,
                sampler: bool = True) -> HostInputs:
    n = context_lengths(cfg)
    tables, nb = block_tables(cfg, n)
    B, Hq, Hkv, D, bs = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    qs, kn, vn, kp, vp = [], [], [], [], []
    for layer in layers:
        qs.append(normal_bf16(_rng(cfg.seed, "q", layer), (B, Hq, D)))
        kn.append(normal_bf16(_rng(cfg.seed, "knew", layer), (B, Hkv, D)))
        vn.append(normal_bf16(_rng(cfg.seed, "vnew", layer), (B, Hkv, D)))
        if pools:
            kp.append(normal_bf16(_rng(cfg.seed, "kpool", layer), (nb, bs, Hkv, D)))
            vp.append(normal_bf16(_rng(cfg.seed, "vpool", layer), (nb, bs, Hkv, D)))
    logits = gumbel = None
    if sampler:
        logits = (_rng(cfg.seed, "logits").standard_normal(size=(B, cfg.vocab), dtype=np.float32)
                  * np.float32(cfg.logit_std))
        gumbel = _rng(cfg.seed, "gumbel").gumbel(size=(B, cfg.vocab)).astype(np.float32)
    t, p, k = sampling_params(cfg)
    return HostInputs(cfg, n, tables, nb, list(layers), qs, kn, vn,
                      kp if pools else None, vp if pools else None,
                      logits, gumbel, t, p, k)


def gumbel_noise(seed: int, shape) -> np.ndarray:
    """Standard Gumbel noise from a named seed (fp64 draw, fp32 result)."""
    return np.random.default_rng([seed, _STREAMS["gumbel"]]).gumbel(size=shape).astype(np.float32)
