"""One decode step as a fixed sequence of library calls.

The step of a paged decode engine (nano-vllm "Model Runner" page, "run
model": prepare, then the model's layers, then the sampler): for each layer
the new token's K/V is stored at its slot and the layer's query attends over
the row's cached positions (split-KV partial step, then the reduce), and
after the last layer the sampler draws one id per row.  This module only
orders the calls; every step of it runs in libpkv's kernels.  The benchmark
times exactly this sequence and the step tests replay it as a HIP graph.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Optional, Sequence

import torch

from . import (cascade_decode_attention, decode_attention_partial,
               decode_attention_partial_store, decode_attention_reduce, kv_store, sample_next_token,
               slot_mapping)


@dataclass
class SamplerArgs:
    logits: torch.Tensor        # fp32 [B, V]
    gumbel: torch.Tensor        # fp32 [B, V]
    temperature: torch.Tensor   # fp32 [B]
    top_p: torch.Tensor         # fp32 [B]
    top_k: torch.Tensor         # int32 [B]
    ids: torch.Tensor           # int32 [B] (out)
    workspace: torch.Tensor


@dataclass
class CascadeArgs:
    prefix_blocks: torch.Tensor  # int32 [P]
    workspace: torch.Tensor


def decode_step(layers: Sequence[tuple], block_tables: torch.Tensor, context_lens: torch.Tensor,
                block_size: int, max_context_len: int, *, out, workspace: torch.Tensor,
                split_tokens: int, sampler: Optional[SamplerArgs] = None, mode: str = "fused",
                slots: Optional[torch.Tensor] = None, cascade: Optional[CascadeArgs] = None,
                mark: Optional[Callable[[str, int], None]] = None) -> None:
    """Enqueue one decode step on the current stream.

    layers   per layer (q, k_cache, v_cache, k_new, v_new): q bf16 [B, Hq, D],
             pools bf16 [NB, bs, Hkv, D], new rows bf16 [B, Hkv, D]
    out      bf16 [B, Hq, D] written by every layer, or one tensor per layer
    mode     "fused": the store runs inside the attention's partial step;
             "unfused": slot mapping once, then per layer store, partial,
             reduce; "cascade": store, then the shared-prefix decode (needs
             `cascade` and `slots`)
    mark     optional callback mark(point, layer) between launches, point in
             "partial", "reduce", "done" (layer) and "sampler", "end" (-1),
             for event timing
    """
    kv_heads = layers[0][1].shape[2]
    stride = block_tables.shape[1]
    if mode in ("unfused", "cascade"):
        if slots is None:
            raise ValueError("unfused and cascade steps need a slots buffer")
        slot_mapping(block_tables, context_lens, block_size, out=slots)
    for li, (q, kc, vc, kn, vn) in enumerate(layers):
        o = out[li] if isinstance(out, (list, tuple)) else out
        if mode != "fused":
            kv_store(kc, vc, kn, vn, slots)
        if mark:
            mark("partial", li)
        if mode == "cascade":
            cascade_decode_attention(q, kc, vc, cascade.prefix_blocks, block_tables, context_lens,
                                     max_context_len, out=o, workspace=cascade.workspace,
                                     split_tokens=split_tokens)
        elif mode == "fused":
            decode_attention_partial_store(q, kc, vc, kn, vn, block_tables, context_lens,
                                           max_context_len, workspace, split_tokens=split_tokens)
        else:
            decode_attention_partial(q, kc, vc, block_tables, context_lens, max_context_len,
                                     workspace, split_tokens=split_tokens)
        if mark:
            mark("reduce", li)
        if mode != "cascade":   # the cascade call includes its own reduce
            decode_attention_reduce(o, context_lens, kv_heads, stride, block_size,
                                    max_context_len, workspace, split_tokens=split_tokens)
        if mark:
            mark("done", li)
    if sampler is not None:
        if mark:
            mark("sampler", -1)
        sample_next_token(sampler.logits, sampler.gumbel, sampler.temperature, sampler.top_p,
                          sampler.top_k, out=sampler.ids, workspace=sampler.workspace)
        if mark:
            mark("end", -1)
