"""CPU oracle of the paged-KV decode step (TEST INFRASTRUCTURE ONLY).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  It wraps ``liboracle.so`` (plain C, built by
``oracle/build.py`` with gcc) through ctypes and shares nothing with the
GPU library.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import LIB_PATH, build as build_oracle

_lib = None


class SampleInfo(ctypes.Structure):
    _fields_ = [
        ("id", ctypes.c_int32),
        ("greedy", ctypes.c_int32),
        ("kept", ctypes.c_int32),
        ("topp_applied", ctypes.c_int32),
        ("tau", ctypes.c_float),
        ("kth", ctypes.c_float),
        ("margin", ctypes.c_double),
    ]


class SampleExtras(ctypes.Structure):
    _fields_ = [
        ("chosen_prob", ctypes.c_double),
        ("top_ids", ctypes.c_int32 * 8),
        ("top_probs", ctypes.c_double * 8),
    ]


def lib():
    """The oracle library.  PKV_ORACLE_LIB names another build of the same
    source to load instead (the tests use it to run the pins against copies
    with planted mistakes, or built with sanitizers)."""
    global _lib
    if _lib is None:
        path = os.environ.get("PKV_ORACLE_LIB") or LIB_PATH
        if path == LIB_PATH and not os.path.exists(LIB_PATH):
            build_oracle()
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.oracle_block_bytes.restype = I64
        L.oracle_block_bytes.argtypes = [I64] * 5
        L.oracle_slot_for_position.restype = I64
        L.oracle_slot_for_position.argtypes = [P, I64, I64, I64]
        L.oracle_slot_mapping.restype = None
        L.oracle_slot_mapping.argtypes = [P, P, I64, P, I64, I64]
        L.oracle_kv_store.restype = ctypes.c_int
        L.oracle_kv_store.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64]
        L.oracle_decode_attention_head.restype = ctypes.c_int
        L.oracle_decode_attention_head.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64, I64,
                                                   ctypes.c_double]
        L.oracle_varlen_attention.restype = ctypes.c_int
        L.oracle_varlen_attention.argtypes = [P, P, P, P, P, I64, P, P, I64, I64, I64, I64, I64,
                                              I64, ctypes.c_double]
        L.oracle_varlen_slot_mapping.restype = None
        L.oracle_varlen_slot_mapping.argtypes = [P, P, I64, P, P, I64, I64]
        L.oracle_decode_attention.restype = ctypes.c_int
        L.oracle_decode_attention.argtypes = [P, P, P, P, P, I64, P, I64, I64, I64, I64, I64, I64,
                                              ctypes.c_double]
        L.oracle_contiguous_attention.restype = ctypes.c_int
        L.oracle_contiguous_attention.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64,
                                                  ctypes.c_double]
        L.oracle_sample_row.restype = ctypes.c_int32
        L.oracle_sample_row.argtypes = [P, P, I64, ctypes.c_float, ctypes.c_float, ctypes.c_int32,
                                        ctypes.POINTER(SampleInfo)]
        L.oracle_sample_row_ex.restype = ctypes.c_int32
        L.oracle_sample_row_ex.argtypes = [P, P, P, I64, ctypes.c_float, ctypes.c_float,
                                           ctypes.c_int32, P, P]
        L.oracle_sample.restype = None
        L.oracle_sample.argtypes = [P, P, P, I64, P, I64, P, P, P, I64, I64]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def block_bytes(num_layers, block_size, num_kv_heads, head_dim, itemsize) -> int:
    return int(lib().oracle_block_bytes(num_layers, block_size, num_kv_heads, head_dim, itemsize))


def slot_for_position(table_row, pos, block_size) -> int:
    t = _c(table_row, np.int32)
    return int(lib().oracle_slot_for_position(_ptr(t), t.size, pos, block_size))


def slot_mapping(block_tables, context_lens, block_size) -> np.ndarray:
    bt = _c(block_tables, np.int32)
    n = _c(context_lens, np.int32)
    out = np.empty(n.shape[0], np.int32)
    lib().oracle_slot_mapping(_ptr(out), _ptr(bt), bt.shape[1], _ptr(n), n.shape[0], block_size)
    return out


def kv_store(k_cache, v_cache, k_new, v_new, slots, block_size) -> int:
    """In place on the uint16 pools k_cache, v_cache [NB, bs, Hkv, D]."""
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    assert k_cache.dtype == np.uint16 and v_cache.dtype == np.uint16
    kn = _c(k_new, np.uint16)
    vn = _c(v_new, np.uint16)
    sl = _c(slots, np.int32)
    nb, bs, hkv, d = k_cache.shape
    assert bs == block_size
    return int(lib().oracle_kv_store(_ptr(k_cache), _ptr(v_cache), _ptr(kn), _ptr(vn), _ptr(sl),
                                     sl.shape[0], hkv, d, bs, nb))


def varlen_attention(q, k_cache, v_cache, block_tables, cu_seqlens_q, cu_seqlens_k,
                     scale=0.0) -> np.ndarray:
    """q uint16 [total_q, Hq, D]; pools uint16 [NB, bs, Hkv, D]; cu_* int32
    [B+1] -> fp64 [total_q, Hq, D] (causal over cached + new tokens)."""
    q = _c(q, np.uint16)
    kc = _c(k_cache, np.uint16)
    vc = _c(v_cache, np.uint16)
    bt = _c(block_tables, np.int32)
    cq = _c(cu_seqlens_q, np.int32)
    ck = _c(cu_seqlens_k, np.int32)
    T, Hq, D = q.shape
    nb, bs, hkv, d2 = kc.shape
    assert d2 == D and cq[-1] == T
    out = np.empty((T, Hq, D), np.float64)
    rc = lib().oracle_varlen_attention(_ptr(out), _ptr(q), _ptr(kc), _ptr(vc), _ptr(bt),
                                       bt.shape[1], _ptr(cq), _ptr(ck), cq.shape[0] - 1, Hq, hkv,
                                       D, bs, nb, float(scale))
    if rc:
        raise ValueError(f"oracle_varlen_attention failed ({rc})")
    return out


def varlen_slot_mapping(block_tables, cu_seqlens_q, cu_seqlens_k, block_size) -> np.ndarray:
    bt = _c(block_tables, np.int32)
    cq = _c(cu_seqlens_q, np.int32)
    ck = _c(cu_seqlens_k, np.int32)
    out = np.empty(int(cq[-1]), np.int32)
    lib().oracle_varlen_slot_mapping(_ptr(out), _ptr(bt), bt.shape[1], _ptr(cq), _ptr(ck),
                                     cq.shape[0] - 1, block_size)
    return out


def decode_attention(q, k_cache, v_cache, block_tables, context_lens, scale=0.0) -> np.ndarray:
    """q uint16 [B, Hq, D]; pools uint16 [NB, bs, Hkv, D] -> fp64 [B, Hq, D]."""
    q = _c(q, np.uint16)
    kc = _c(k_cache, np.uint16)
    vc = _c(v_cache, np.uint16)
    bt = _c(block_tables, np.int32)
    n = _c(context_lens, np.int32)
    B, Hq, D = q.shape
    nb, bs, hkv, d2 = kc.shape
    assert d2 == D
    out = np.empty((B, Hq, D), np.float64)
    rc = lib().oracle_decode_attention(_ptr(out), _ptr(q), _ptr(kc), _ptr(vc), _ptr(bt),
                                       bt.shape[1], _ptr(n), B, Hq, hkv, D, bs, nb, float(scale))
    if rc:
        raise ValueError(f"oracle_decode_attention failed ({rc})")
    return out


def decode_attention_head(q_head, k_cache, v_cache, table_row, context_len, kv_head,
                          scale) -> np.ndarray:
    """One (row, query head) output in fp64; scale must be explicit (> 0)."""
    qh = _c(q_head, np.uint16)
    kc = k_cache if k_cache.flags.c_contiguous else np.ascontiguousarray(k_cache)
    vc = v_cache if v_cache.flags.c_contiguous else np.ascontiguousarray(v_cache)
    tr = _c(table_row, np.int32)
    nb, bs, hkv, D = kc.shape
    out = np.empty(D, np.float64)
    rc = lib().oracle_decode_attention_head(_ptr(out), _ptr(qh), _ptr(kc), _ptr(vc), _ptr(tr),
                                            int(context_len), hkv, int(kv_head), D, bs, nb,
                                            float(scale))
    if rc:
        raise ValueError(f"oracle_decode_attention_head failed ({rc})")
    return out


def contiguous_attention(q, k, v, context_lens, scale=0.0) -> np.ndarray:
    """Cache layout [B, T, Hkv, D] (uint16) -> fp64 [B, Hq, D]."""
    q = _c(q, np.uint16)
    k = _c(k, np.uint16)
    v = _c(v, np.uint16)
    n = _c(context_lens, np.int32)
    B, Hq, D = q.shape
    _, T, hkv, _ = k.shape
    out = np.empty((B, Hq, D), np.float64)
    rc = lib().oracle_contiguous_attention(_ptr(out), _ptr(q), _ptr(k), _ptr(v), _ptr(n), B, T,
                                           Hq, hkv, D, float(scale))
    if rc:
        raise ValueError(f"oracle_contiguous_attention failed ({rc})")
    return out


def sample_row(logits, gumbel, temperature, top_p, top_k):
    z = _c(logits, np.float32)
    g = _c(gumbel, np.float32)
    info = SampleInfo()
    lib().oracle_sample_row(_ptr(z), _ptr(g), z.shape[0], float(temperature), float(top_p),
                            int(top_k), ctypes.byref(info))
    return info


def sample_row_ex(logits, gumbel, temperature, top_p, top_k, mask=None):
    """One row with the vocabulary mask (uint8/bool [V], nonzero = allowed,
    or None) and the extra outputs; returns (SampleInfo, SampleExtras)."""
    z = _c(logits, np.float32)
    g = _c(gumbel, np.float32)
    m = None if mask is None else _c(mask, np.uint8)
    info, extras = SampleInfo(), SampleExtras()
    lib().oracle_sample_row_ex(_ptr(z), _ptr(g), None if m is None else _ptr(m), z.shape[0],
                               float(temperature), float(top_p), int(top_k),
                               ctypes.byref(info), ctypes.byref(extras))
    return info, extras


def sample(logits, gumbel, temperature, top_p, top_k):
    """Returns (ids int32 [B], list of SampleInfo)."""
    z = _c(logits, np.float32)
    g = _c(gumbel, np.float32)
    t = _c(temperature, np.float32)
    p = _c(top_p, np.float32)
    k = _c(top_k, np.int32)
    B, V = z.shape
    ids = np.empty(B, np.int32)
    infos = (SampleInfo * B)()
    lib().oracle_sample(_ptr(ids), ctypes.cast(infos, ctypes.c_void_p), _ptr(z), V, _ptr(g), V,
                        _ptr(t), _ptr(p), _ptr(k), B, V)
    return ids, list(infos)
