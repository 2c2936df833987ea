"""paged_kv_decode_store_amd - MI355X-native paged-KV decode step.

A thin Python binding over libpkv.so (include/pkv.h).  Each function checks
tensor dtypes/devices, passes raw device pointers and the current HIP stream
to the C ABI, and raises on a non-zero status.  Every step of the path runs
in the library's HIP kernels; PyTorch only provides device memory and the
stream.  There is no CPU fallback: importing the package does not need a
GPU, but every call does.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib
from ._lib import (PKV_DEVERR_BLOCK_ID, PKV_DEVERR_CONTEXT_LEN, PKV_DEVERR_SEQLENS,
                   PKV_DEVERR_SLOT, PKV_DEVERR_WAIT, PkvError,
                   check, lib)

__all__ = [
    "slot_mapping", "kv_store", "paged_decode_attention", "decode_attention_partial",
    "decode_attention_reduce", "decode_workspace_bytes", "decode_split_tokens",
    "paged_decode_attention_store", "decode_attention_partial_store",
    "cascade_decode_attention", "cascade_workspace_bytes",
    "varlen_slot_mapping", "varlen_paged_attention",
    "sample_next_token", "sample_next_token_ex", "sampler_workspace_bytes", "PkvError",
    "varlen_split_tokens", "varlen_workspace_bytes",
    "set_error_word", "set_wait_limit", "paged_decode_attention_store_noalloc", "PKV_DEVERR_SLOT", "PKV_DEVERR_BLOCK_ID",
    "PKV_DEVERR_CONTEXT_LEN", "PKV_DEVERR_SEQLENS", "PKV_DEVERR_WAIT",
]


def set_error_word(word: Optional[torch.Tensor]) -> None:
    """Report device-side contract violations (PKV_DEVERR_* bits) into
    `word`, a one-element int32 GPU tensor the caller zeroes and reads; None
    stops reporting.  Applies to later calls from this host thread."""
    if word is None:
        check(lib().pkv_set_error_word(None), "pkv_set_error_word")
        return
    if word.numel() < 1:
        raise ValueError("word must hold at least one element")
    check(lib().pkv_set_error_word(_dev(word, "word", torch.int32)), "pkv_set_error_word")


def set_wait_limit(polls: int) -> None:
    """Poll cap of the kernels' bounded waits for this host thread (0 = the
    default); a test hook that makes the waits give up and report."""
    check(lib().pkv_set_wait_limit(int(polls)), "pkv_set_wait_limit")


def _stream():
    return ctypes_ptr(torch.cuda.current_stream().cuda_stream)


def ctypes_ptr(x: int):
    return None if x == 0 else x


def _dev(t: torch.Tensor, name: str, dtype) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _packed(t: torch.Tensor, name: str):
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def probe_stream_read(buf: torch.Tensor, sink: torch.Tensor, workgroups: int = 0) -> None:
    """Streaming-read probe over the bytes of `buf` (a multiple of 16); sink:
    int32 [64] on the same device.  Timing is the caller's."""
    if not buf.is_cuda:
        raise ValueError("buf must be a GPU tensor")
    _packed(buf, "buf")
    nbytes = buf.numel() * buf.element_size()
    _lib.check(_lib.lib().pkv_probe_stream_read(
        buf.data_ptr(), nbytes, _dev(sink, "sink", torch.int32), workgroups, _stream()),
        "probe_stream_read")


def device_info(device: int = 0) -> dict:
    """Properties of a device as the HIP runtime reports them."""
    info = _lib.DeviceInfo()
    _lib.check(_lib.lib().pkv_get_device_info(device, ctypes.byref(info)), "device_info")
    out = {f: getattr(info, f) for f, _ in _lib.DeviceInfo._fields_ if f != "pad"}
    out["name"] = info.name.decode(errors="replace")
    out["arch"] = info.arch.decode(errors="replace")
    return out


def slot_mapping(block_tables: torch.Tensor, context_lens: torch.Tensor, block_size: int,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """int32 [B] slot of each row's new token (position context_len - 1)."""
    B = context_lens.shape[0]
    _packed(block_tables, "block_tables")
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=context_lens.device)
    check(lib().pkv_slot_mapping(_dev(out, "out", torch.int32),
                                 _dev(block_tables, "block_tables", torch.int32),
                                 block_tables.shape[1],
                                 _dev(context_lens, "context_lens", torch.int32), B, block_size,
                                 _stream()), "pkv_slot_mapping")
    return out


def kv_store(k_cache: torch.Tensor, v_cache: torch.Tensor, k_new: torch.Tensor,
             v_new: torch.Tensor, slots: torch.Tensor) -> None:
    """In-place store of k_new/v_new [T, Hkv, D] rows into pools
    [NB, bs, Hkv, D] at slots [T]."""
    nb, bs, hkv, d = k_cache.shape
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _packed(t, name)
    assert v_cache.shape == k_cache.shape
    T = k_new.shape[0]
    if k_new.shape[1:] != (hkv, d) or v_new.shape[1:] != (hkv, d):
        raise ValueError("k_new/v_new must be [T, Hkv, D] matching the pools")
    if k_new.stride(1) != d or k_new.stride(2) != 1 or v_new.stride() != k_new.stride():
        raise ValueError("k_new/v_new rows must be packed [Hkv, D] with equal strides")
    check(lib().pkv_kv_store(_dev(k_cache, "k_cache", torch.bfloat16),
                             _dev(v_cache, "v_cache", torch.bfloat16),
                             _dev(k_new, "k_new", torch.bfloat16),
                             _dev(v_new, "v_new", torch.bfloat16),
                             _dev(slots, "slots", torch.int32), T, hkv, d, k_new.stride(0), bs, nb,
                             _stream()), "pkv_kv_store")


def decode_split_tokens(batch: int, num_q_heads: int, num_kv_heads: int, max_context_len: int,
                        split_tokens: int = 0) -> int:
    s = int(lib().pkv_decode_split_tokens(batch, num_q_heads, num_kv_heads, max_context_len,
                                          split_tokens))
    if s == 0 and split_tokens != 0:   # the library answers 0 for a split it rejects
        raise _lib.PkvError(_lib.PKV_ERR_INVALID_ARG, "pkv_decode_split_tokens")
    return s


def decode_workspace_bytes(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                           max_context_len: int, split_tokens: int = 0) -> int:
    return int(lib().pkv_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim,
                                                max_context_len, split_tokens))


def _workspace(nbytes: int, device, workspace):
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    if workspace.dtype != torch.uint8 or not workspace.is_cuda:
        raise TypeError("workspace must be a uint8 GPU tensor")
    return workspace


def _attn_shapes(q, k_cache, block_tables):
    B, Hq, D = q.shape
    nb, bs, hkv, d2 = k_cache.shape
    if d2 != D:
        raise ValueError("q and cache head_dim differ")
    if q.stride(2) != 1 or q.stride(1) != D:
        raise ValueError("q rows must be packed [Hq, D]")
    _packed(block_tables, "block_tables")
    return B, Hq, D, nb, bs, hkv


def decode_attention_partial(q, k_cache, v_cache, block_tables, context_lens, max_context_len,
                             workspace, scale: float = 0.0, split_tokens: int = 0) -> None:
    B, Hq, D, nb, bs, hkv = _attn_shapes(q, k_cache, block_tables)
    check(lib().pkv_decode_attention_partial(
        _dev(q, "q", torch.bfloat16), q.stride(0), _dev(k_cache, "k_cache", torch.bfloat16),
        _dev(v_cache, "v_cache", torch.bfloat16), _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1], _dev(context_lens, "context_lens", torch.int32), B, Hq, hkv, D, bs,
        nb, max_context_len, scale, split_tokens, _dev(workspace, "workspace", torch.uint8),
        workspace.numel(), _stream()), "pkv_decode_attention_partial")


def decode_attention_reduce(out, context_lens, num_kv_heads, block_table_stride, block_size,
                            max_context_len, workspace, split_tokens: int = 0) -> None:
    B, Hq, D = out.shape
    if out.stride(2) != 1 or out.stride(1) != D:
        raise ValueError("out rows must be packed [Hq, D]")
    check(lib().pkv_decode_attention_reduce(
        _dev(out, "out", torch.bfloat16), out.stride(0),
        _dev(context_lens, "context_lens", torch.int32), B, Hq, num_kv_heads, D,
        block_table_stride, block_size, max_context_len, split_tokens,
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream()),
        "pkv_decode_attention_reduce")


def paged_decode_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           block_tables: torch.Tensor, context_lens: torch.Tensor,
                           max_context_len: int, scale: float = 0.0, split_tokens: int = 0,
                           out: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16 [B, Hq, D] attention of each row's query over its n_b cached
    positions (context_lens, new token included)."""
    B, Hq, D, nb, bs, hkv = _attn_shapes(q, k_cache, block_tables)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=q.device)
    ws = _workspace(decode_workspace_bytes(B, Hq, hkv, D, max_context_len, split_tokens),
                    q.device, workspace)
    check(lib().pkv_paged_decode_attention(
        _dev(out, "out", torch.bfloat16), out.stride(0), _dev(q, "q", torch.bfloat16), q.stride(0),
        _dev(k_cache, "k_cache", torch.bfloat16), _dev(v_cache, "v_cache", torch.bfloat16),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), B, Hq, hkv, D, bs, nb, max_context_len,
        scale, split_tokens, ws.data_ptr(), ws.numel(), _stream()), "pkv_paged_decode_attention")
    return out


def cascade_workspace_bytes(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                            max_context_len: int, num_prefix_blocks: int, block_size: int,
                            split_tokens: int = 0) -> int:
    n = lib().pkv_cascade_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim,
                                          max_context_len, num_prefix_blocks, block_size,
                                          split_tokens)
    if n == 0:
        raise ValueError("invalid cascade workspace query (shapes or split_tokens)")
    return n


def cascade_decode_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                             prefix_blocks: torch.Tensor, block_tables: torch.Tensor,
                             context_lens: torch.Tensor, max_context_len: int,
                             scale: float = 0.0, split_tokens: int = 0,
                             out: Optional[torch.Tensor] = None,
                             workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode attention for rows whose first len(prefix_blocks) blocks are the
    shared blocks prefix_blocks (int32): the prefix is read once for all
    rows.  Same result as paged_decode_attention over the whole rows."""
    B, Hq, D, nb, bs, hkv = _attn_shapes(q, k_cache, block_tables)
    if prefix_blocks.dim() != 1 or prefix_blocks.numel() == 0:
        raise ValueError("prefix_blocks must be a non-empty 1-D int32 tensor")
    npb = prefix_blocks.numel()
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=q.device)
    ws = _workspace(cascade_workspace_bytes(B, Hq, hkv, D, max_context_len, npb, bs, split_tokens),
                    q.device, workspace)
    check(lib().pkv_cascade_decode_attention(
        _dev(out, "out", torch.bfloat16), out.stride(0), _dev(q, "q", torch.bfloat16), q.stride(0),
        _dev(k_cache, "k_cache", torch.bfloat16), _dev(v_cache, "v_cache", torch.bfloat16),
        _dev(prefix_blocks, "prefix_blocks", torch.int32), npb,
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), B, Hq, hkv, D, bs, nb, max_context_len,
        scale, split_tokens, ws.data_ptr(), ws.numel(), _stream()), "pkv_cascade_decode_attention")
    return out


def _new_rows(k_new, v_new, hkv, D):
    if k_new.shape[1:] != (hkv, D) or v_new.shape[1:] != (hkv, D):
        raise ValueError("k_new/v_new must be [B, Hkv, D] matching the pools")
    if k_new.stride(1) != D or k_new.stride(2) != 1 or v_new.stride() != k_new.stride():
        raise ValueError("k_new/v_new rows must be packed [Hkv, D] with equal strides")
    return k_new.stride(0)


def decode_attention_partial_store(q, k_cache, v_cache, k_new, v_new, block_tables, context_lens,
                                   max_context_len, workspace, scale: float = 0.0,
                                   split_tokens: int = 0) -> None:
    """Fused store + partial step: row b's new position (context_lens[b]-1)
    takes its K/V from k_new/v_new [B, Hkv, D] and is written to the pools."""
    B, Hq, D, nb, bs, hkv = _attn_shapes(q, k_cache, block_tables)
    ns = _new_rows(k_new, v_new, hkv, D)
    check(lib().pkv_decode_attention_partial_store(
        _dev(q, "q", torch.bfloat16), q.stride(0), _dev(k_cache, "k_cache", torch.bfloat16),
        _dev(v_cache, "v_cache", torch.bfloat16), _dev(k_new, "k_new", torch.bfloat16),
        _dev(v_new, "v_new", torch.bfloat16), ns, _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1], _dev(context_lens, "context_lens", torch.int32), B, Hq, hkv, D, bs,
        nb, max_context_len, scale, split_tokens, _dev(workspace, "workspace", torch.uint8),
        workspace.numel(), _stream()), "pkv_decode_attention_partial_store")


def paged_decode_attention_store(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                 k_new: torch.Tensor, v_new: torch.Tensor,
                                 block_tables: torch.Tensor, context_lens: torch.Tensor,
                                 max_context_len: int, scale: float = 0.0, split_tokens: int = 0,
                                 out: Optional[torch.Tensor] = None,
                                 workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Fused decode step for one layer: store each row's new K/V at its slot
    and attend over the n_b positions; equals slot_mapping + kv_store +
    paged_decode_attention."""
    B, Hq, D, nb, bs, hkv = _attn_shapes(q, k_cache, block_tables)
    ns = _new_rows(k_new, v_new, hkv, D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=q.device)
    ws = _workspace(decode_workspace_bytes(B, Hq, hkv, D, max_context_len, split_tokens),
                    q.device, workspace)
    check(lib().pkv_paged_decode_attention_store(
        _dev(out, "out", torch.bfloat16), out.stride(0), _dev(q, "q", torch.bfloat16), q.stride(0),
        _dev(k_cache, "k_cache", torch.bfloat16), _dev(v_cache, "v_cache", torch.bfloat16),
        _dev(k_new, "k_new", torch.bfloat16), _dev(v_new, "v_new", torch.bfloat16), ns,
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), B, Hq, hkv, D, bs, nb, max_context_len,
        scale, split_tokens, ws.data_ptr(), ws.numel(), _stream()),
        "pkv_paged_decode_attention_store")
    return out


def paged_decode_attention_store_noalloc(q: torch.Tensor, k_cache: torch.Tensor,
                                         v_cache: torch.Tensor, k_new: torch.Tensor,
                                         v_new: torch.Tensor, block_tables: torch.Tensor,
                                         context_lens: torch.Tensor, max_context_len: int,
                                         out: torch.Tensor, scale: float = 0.0,
                                         split_tokens: int = 0) -> torch.Tensor:
    """paged_decode_attention_store without a workspace: the partials live
    in the library's fixed device array (PKV_STATIC_SCRATCH_BYTES), so the
    call allocates nothing (the caller passes `out`).  Calls overlapping in
    time on one GPU race on that array."""
    B, Hq, D, nb, bs, hkv = _attn_shapes(q, k_cache, block_tables)
    ns = _new_rows(k_new, v_new, hkv, D)
    check(lib().pkv_paged_decode_attention_store_noalloc(
        _dev(out, "out", torch.bfloat16), out.stride(0), _dev(q, "q", torch.bfloat16), q.stride(0),
        _dev(k_cache, "k_cache", torch.bfloat16), _dev(v_cache, "v_cache", torch.bfloat16),
        _dev(k_new, "k_new", torch.bfloat16), _dev(v_new, "v_new", torch.bfloat16), ns,
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), B, Hq, hkv, D, bs, nb, max_context_len,
        scale, split_tokens, _stream()), "pkv_paged_decode_attention_store_noalloc")
    return out


def sampler_workspace_bytes(batch: int, vocab: int) -> int:
    return int(lib().pkv_sampler_workspace_bytes(batch, vocab))


def sample_next_token(logits: torch.Tensor, gumbel: torch.Tensor, temperature: torch.Tensor,
                      top_p: torch.Tensor, top_k: torch.Tensor,
                      out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """int32 [B] next-token ids; each row's own temperature, top_p and top_k
    decide its filters."""
    B, V = logits.shape
    if logits.stride(1) != 1 or gumbel.stride(1) != 1 or gumbel.shape != logits.shape:
        raise ValueError("logits/gumbel must be [B, V] with unit element stride")
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=logits.device)
    ws = _workspace(sampler_workspace_bytes(B, V), logits.device, workspace)
    check(lib().pkv_sample_next_token(
        _dev(out, "out", torch.int32), _dev(logits, "logits", torch.float32), logits.stride(0),
        _dev(gumbel, "gumbel", torch.float32), gumbel.stride(0),
        _dev(temperature, "temperature", torch.float32), _dev(top_p, "top_p", torch.float32),
        _dev(top_k, "top_k", torch.int32), B, V, ws.data_ptr(), ws.numel(), _stream()),
        "pkv_sample_next_token")
    return out


def sample_next_token_ex(logits: torch.Tensor, gumbel: torch.Tensor, temperature: torch.Tensor,
                         top_p: torch.Tensor, top_k: torch.Tensor,
                         mask: Optional[torch.Tensor] = None,
                         extras: bool = True, out: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None):
    """Next-token ids with the vocabulary mask (uint8/bool [B, V], nonzero =
    allowed, or None) and, when extras is true, the drawn token's
    probability [B] and the top-8 ids / probabilities [B, 8].  Returns ids,
    or (ids, prob, top_ids, top_probs)."""
    B, V = logits.shape
    if logits.stride(1) != 1 or gumbel.stride(1) != 1 or gumbel.shape != logits.shape:
        raise ValueError("logits/gumbel must be [B, V] with unit element stride")
    mptr, mstride = None, 0
    if mask is not None:
        if mask.dtype == torch.bool:
            mask = mask.view(torch.uint8)
        if mask.shape != logits.shape or mask.stride(1) != 1:
            raise ValueError("mask must be [B, V] with unit element stride")
        mptr, mstride = _dev(mask, "mask", torch.uint8), mask.stride(0)
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=logits.device)
    prob = top_ids = top_probs = None
    if extras:
        prob = torch.empty(B, dtype=torch.float32, device=logits.device)
        top_ids = torch.empty((B, 8), dtype=torch.int32, device=logits.device)
        top_probs = torch.empty((B, 8), dtype=torch.float32, device=logits.device)
    ws = _workspace(sampler_workspace_bytes(B, V), logits.device, workspace)
    check(lib().pkv_sample_next_token_ex(
        _dev(out, "out", torch.int32), _dev(logits, "logits", torch.float32), logits.stride(0),
        _dev(gumbel, "gumbel", torch.float32), gumbel.stride(0), mptr, mstride,
        _dev(temperature, "temperature", torch.float32), _dev(top_p, "top_p", torch.float32),
        _dev(top_k, "top_k", torch.int32), B, V,
        None if prob is None else prob.data_ptr(), None if top_ids is None else top_ids.data_ptr(),
        None if top_probs is None else top_probs.data_ptr(), ws.data_ptr(), ws.numel(), _stream()),
        "pkv_sample_next_token_ex")
    if not extras:
        return out
    return out, prob, top_ids, top_probs


def varlen_slot_mapping(block_tables: torch.Tensor, cu_seqlens_q: torch.Tensor,
                        cu_seqlens_k: torch.Tensor, max_seqlen_q: int, block_size: int,
                        total_q: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """int32 [total_q] slots of the new tokens of a varlen batch."""
    B = cu_seqlens_q.numel() - 1
    if out is None:
        out = torch.empty(total_q, dtype=torch.int32, device=block_tables.device)
    _packed(block_tables, "block_tables")
    check(lib().pkv_varlen_slot_mapping(
        _dev(out, "slot_mapping", torch.int32), _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1], _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32),
        _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32), B, max_seqlen_q, block_size, _stream()),
        "pkv_varlen_slot_mapping")
    return out


def varlen_split_tokens(batch: int, num_q_heads: int, num_kv_heads: int, max_seqlen_q: int,
                        max_seqlen_k: int, split_tokens: int = 0) -> int:
    return int(lib().pkv_varlen_split_tokens(batch, num_q_heads, num_kv_heads, max_seqlen_q,
                                             max_seqlen_k, split_tokens))


def varlen_workspace_bytes(total_q: int, batch: int, num_q_heads: int, num_kv_heads: int,
                           head_dim: int, max_seqlen_q: int, max_seqlen_k: int,
                           split_tokens: int = 0) -> int:
    return int(lib().pkv_varlen_workspace_bytes(total_q, batch, num_q_heads, num_kv_heads,
                                                head_dim, max_seqlen_q, max_seqlen_k,
                                                split_tokens))


def varlen_paged_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           block_tables: torch.Tensor, cu_seqlens_q: torch.Tensor,
                           cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int,
                           scale: float = 0.0, split_tokens: int = 0,
                           out: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16 [total_q, Hq, D]: each new token of each sequence attends causally
    to the sequence's cached tokens and to the new tokens up to itself."""
    T, Hq, D = q.shape
    nb, bs, hkv, d2 = k_cache.shape
    if d2 != D or v_cache.shape != k_cache.shape:
        raise ValueError("pools must be [NB, bs, Hkv, D] matching q")
    if q.stride(2) != 1 or q.stride(1) != D:
        raise ValueError("q rows must be packed [Hq, D]")
    _packed(k_cache, "k_cache")
    _packed(v_cache, "v_cache")
    _packed(block_tables, "block_tables")
    B = cu_seqlens_q.numel() - 1
    if out is None:
        out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=q.device)
    need = varlen_workspace_bytes(T, B, Hq, hkv, D, max_seqlen_q, max_seqlen_k, split_tokens)
    ws = _workspace(need, q.device, workspace) if need else None
    check(lib().pkv_varlen_paged_attention(
        _dev(out, "out", torch.bfloat16), out.stride(0), _dev(q, "q", torch.bfloat16), q.stride(0),
        _dev(k_cache, "k_cache", torch.bfloat16), _dev(v_cache, "v_cache", torch.bfloat16),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32),
        _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32), B, T, Hq, hkv, D, bs, nb, max_seqlen_q,
        max_seqlen_k, scale, split_tokens,
        _dev(ws, "workspace", torch.uint8) if ws is not None else None,
        ws.numel() if ws is not None else 0, _stream()), "pkv_varlen_paged_attention")
    return out
