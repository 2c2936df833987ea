"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every entry point include/pkv.h declares, and
refuse bad arguments on the host, before any HIP call.  No test here passes
a set of arguments that would reach a kernel launch: every call below fails
validation.
"""
import ctypes
import os
import re

import pytest

import paged_kv_decode_store_amd as pkv
from paged_kv_decode_store_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 4096  # a non-null, 256-byte aligned fake device address; never dereferenced


def declared_functions():
    text = open(os.path.join(ROOT, "include", "pkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = _lib.lib()
    names = declared_functions()
    assert len(names) == 26, names
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.PROTOTYPES)


def test_probe_arguments_are_checked_before_any_launch():
    """The streaming-read probe refuses a length that is not a multiple of 16,
    misaligned buffers and a negative workgroup count (no kernel runs here)."""
    L = _lib.lib()
    assert L.pkv_probe_stream_read(FAKE, 24, FAKE, 0, None) == _lib.PKV_ERR_INVALID_ARG
    assert L.pkv_probe_stream_read(FAKE + 8, 32, FAKE, 0, None) == _lib.PKV_ERR_INVALID_ARG
    assert L.pkv_probe_stream_read(FAKE, 32, FAKE + 2, 0, None) == _lib.PKV_ERR_INVALID_ARG
    assert L.pkv_probe_stream_read(FAKE, 32, FAKE, -1, None) == _lib.PKV_ERR_INVALID_ARG
    assert L.pkv_probe_stream_read(None, 0, None, 0, None) == _lib.PKV_OK
    assert L.pkv_get_device_info(0, None) == _lib.PKV_ERR_INVALID_ARG


def test_error_word_setting_is_per_thread_and_checked():
    """Host side of the device error word: a misaligned word is refused,
    a set word is returned by the getter, NULL stops reporting, and another
    host thread keeps its own setting.  (No kernel runs here.)"""
    import threading
    L = _lib.lib()
    assert L.pkv_set_error_word(FAKE + 2) == _lib.PKV_ERR_INVALID_ARG
    assert L.pkv_set_error_word(FAKE) == _lib.PKV_OK
    assert L.pkv_get_error_word() == FAKE
    seen = []
    th = threading.Thread(target=lambda: seen.append(L.pkv_get_error_word()))
    th.start()
    th.join()
    assert seen == [None]
    assert L.pkv_set_error_word(None) == _lib.PKV_OK
    assert L.pkv_get_error_word() is None
    assert L.pkv_set_wait_limit(5) == _lib.PKV_OK
    assert L.pkv_set_wait_limit(0) == _lib.PKV_OK


def test_status_strings():
    L = _lib.lib()
    assert L.pkv_status_string(0) == b"ok"
    for code in (-1, -2, -3, -4):
        assert L.pkv_status_string(code) not in (b"ok", b"unknown status")


def test_slot_mapping_validation():
    L = _lib.lib()
    assert L.pkv_slot_mapping(None, FAKE, 4, FAKE, 3, 256, None) == _lib.PKV_ERR_INVALID_ARG
    assert L.pkv_slot_mapping(FAKE, FAKE, 0, FAKE, 3, 256, None) == _lib.PKV_ERR_INVALID_ARG
    assert L.pkv_slot_mapping(FAKE, FAKE, 4, FAKE, 3, 100, None) == _lib.PKV_ERR_UNSUPPORTED
    assert L.pkv_slot_mapping(FAKE, FAKE, 4, FAKE, -1, 256, None) == _lib.PKV_ERR_INVALID_ARG
    # an empty batch is a no-op, not an error, and launches nothing
    assert L.pkv_slot_mapping(None, None, 4, None, 0, 256, None) == _lib.PKV_OK


def test_kv_store_validation():
    L = _lib.lib()
    ok = dict(k=FAKE, v=FAKE, kn=FAKE, vn=FAKE, s=FAKE, T=4, H=8, D=128, st=0, bs=256, nb=10)

    def call(**kw):
        a = dict(ok, **kw)
        return L.pkv_kv_store(a["k"], a["v"], a["kn"], a["vn"], a["s"], a["T"], a["H"], a["D"],
                              a["st"], a["bs"], a["nb"], None)

    assert call(k=None) == _lib.PKV_ERR_INVALID_ARG
    assert call(kn=FAKE + 2) == _lib.PKV_ERR_INVALID_ARG          # misaligned bf16
    assert call(D=100) == _lib.PKV_ERR_UNSUPPORTED
    assert call(bs=96) == _lib.PKV_ERR_UNSUPPORTED
    assert call(st=8 * 128 - 8) == _lib.PKV_ERR_INVALID_ARG      # stride below a row
    assert call(nb=0) == _lib.PKV_ERR_INVALID_ARG
    assert call(T=0, k=None, v=None, kn=None, vn=None, s=None) == _lib.PKV_OK
    assert b"aligned" in L.pkv_last_error() or True


def _attn_call(L, **kw):
    a = dict(out=FAKE, ostride=0, q=FAKE, qstride=0, k=FAKE, v=FAKE, bt=FAKE, bts=16, lens=FAKE,
             B=64, Hq=16, Hkv=8, D=128, bs=256, nb=600, maxlen=4096, scale=0.0, split=0,
             ws=FAKE, wsb=0)
    a.update(kw)
    return L.pkv_paged_decode_attention(a["out"], a["ostride"], a["q"], a["qstride"], a["k"],
                                        a["v"], a["bt"], a["bts"], a["lens"], a["B"], a["Hq"],
                                        a["Hkv"], a["D"], a["bs"], a["nb"], a["maxlen"],
                                        a["scale"], a["split"], a["ws"], a["wsb"], None)


def test_attention_validation():
    L = _lib.lib()
    need = L.pkv_decode_workspace_bytes(64, 16, 8, 128, 4096, 0)
    assert need > 0
    # every case below fails one check; the last one fails only the workspace size
    assert _attn_call(L, q=None, wsb=need) == _lib.PKV_ERR_INVALID_ARG
    assert _attn_call(L, out=None, wsb=need) == _lib.PKV_ERR_INVALID_ARG
    assert _attn_call(L, k=FAKE + 8, wsb=need) == _lib.PKV_ERR_INVALID_ARG
    assert _attn_call(L, D=96, wsb=need) == _lib.PKV_ERR_UNSUPPORTED
    assert _attn_call(L, bs=8, wsb=need) == _lib.PKV_ERR_UNSUPPORTED
    assert _attn_call(L, Hq=12, wsb=need) == _lib.PKV_ERR_INVALID_ARG  # 12 % 8 != 0
    assert _attn_call(L, split=100, wsb=need) == _lib.PKV_ERR_INVALID_ARG
    assert _attn_call(L, scale=float("nan"), wsb=need) == _lib.PKV_ERR_INVALID_ARG
    assert _attn_call(L, qstride=16 * 128 - 8, wsb=need) == _lib.PKV_ERR_INVALID_ARG
    assert _attn_call(L, ws=FAKE + 16, wsb=need) == _lib.PKV_ERR_WORKSPACE
    assert _attn_call(L, ws=None, wsb=need) == _lib.PKV_ERR_WORKSPACE
    assert _attn_call(L, wsb=need - 1) == _lib.PKV_ERR_WORKSPACE
    assert b"workspace too small" in L.pkv_last_error()


def test_workspace_and_split_queries():
    L = _lib.lib()
    for (B, Hq, Hkv, ml) in [(64, 16, 8, 4096), (8, 64, 8, 131072), (4, 16, 16, 513),
                             (32, 48, 8, 2048), (1, 1, 1, 1)]:
        s = L.pkv_decode_split_tokens(B, Hq, Hkv, ml, 0)
        assert s >= 64 and s % 64 == 0
        assert L.pkv_decode_split_tokens(B, Hq, Hkv, ml, 128) == 128
    assert L.pkv_decode_split_tokens(4, 4, 4, 100, 100) == 0  # not a multiple of 64
    # the binding turns that 0 into an error instead of passing it on (where
    # 0 would mean the automatic split)
    with pytest.raises(_lib.PkvError):
        pkv.decode_split_tokens(64, 16, 8, 4096, 288)
    assert pkv.decode_split_tokens(64, 16, 8, 4096, 320) == 320
    # workspace: [B][Hq][S][D] + [B][Hq][S][2] fp32, each 256-byte aligned
    B, Hq, Hkv, D, ml, split = 3, 4, 2, 64, 1000, 128
    S = (ml + split - 1) // split
    o = B * Hq * S * D * 4
    m = B * Hq * S * 2 * 4
    expect = ((o + 255) // 256) * 256 + ((m + 255) // 256) * 256
    assert L.pkv_decode_workspace_bytes(B, Hq, Hkv, D, ml, split) == expect
    assert L.pkv_decode_workspace_bytes(B, Hq, Hkv, D, ml, 100) == 0
    assert L.pkv_sampler_workspace_bytes(64, 151936) > 64 * 2048 * 12
    assert L.pkv_sampler_workspace_bytes(1, 0) == 0


def test_sampler_validation():
    L = _lib.lib()
    need = L.pkv_sampler_workspace_bytes(8, 1000)

    def call(**kw):
        a = dict(ids=FAKE, z=FAKE, zs=0, g=FAKE, gs=0, t=FAKE, p=FAKE, k=FAKE, B=8, V=1000,
                 ws=FAKE, wsb=need)
        a.update(kw)
        return L.pkv_sample_next_token(a["ids"], a["z"], a["zs"], a["g"], a["gs"], a["t"], a["p"],
                                       a["k"], a["B"], a["V"], a["ws"], a["wsb"], None)

    assert call(z=None) == _lib.PKV_ERR_INVALID_ARG
    assert call(t=FAKE + 2) == _lib.PKV_ERR_INVALID_ARG
    assert call(V=0) == _lib.PKV_ERR_UNSUPPORTED
    assert call(V=(1 << 24) + 1) == _lib.PKV_ERR_UNSUPPORTED
    assert call(B=65536) == _lib.PKV_ERR_INVALID_ARG
    assert call(zs=999) == _lib.PKV_ERR_INVALID_ARG
    assert call(wsb=need - 1) == _lib.PKV_ERR_WORKSPACE
    assert call(B=0, ids=None, z=None, g=None) == _lib.PKV_OK


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    import paged_kv_decode_store_amd as pkv

    bt = torch.zeros((2, 2), dtype=torch.int32)
    lens = torch.ones(2, dtype=torch.int32)
    with pytest.raises(ValueError):
        pkv.slot_mapping(bt, lens, 256, out=torch.empty(2, dtype=torch.int32))


def test_fused_attention_validation():
    L = _lib.lib()
    need = L.pkv_decode_workspace_bytes(64, 16, 8, 128, 4096, 0)

    def call(**kw):
        a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, kn=FAKE, vn=FAKE, ns=0, bt=FAKE, lens=FAKE,
                 ws=FAKE, wsb=need)
        a.update(kw)
        return L.pkv_paged_decode_attention_store(a["out"], 0, a["q"], 0, a["k"], a["v"], a["kn"],
                                                  a["vn"], a["ns"], a["bt"], 16, a["lens"], 64, 16,
                                                  8, 128, 256, 600, 4096, 0.0, 0, a["ws"], a["wsb"],
                                                  None)

    assert call(kn=None) == _lib.PKV_ERR_INVALID_ARG
    assert call(vn=FAKE + 4) == _lib.PKV_ERR_INVALID_ARG
    assert call(ns=8 * 128 - 8) == _lib.PKV_ERR_INVALID_ARG
    assert call(out=None) == _lib.PKV_ERR_INVALID_ARG
    assert call(wsb=need - 1) == _lib.PKV_ERR_WORKSPACE


def test_noalloc_attention_validation():
    """The no-allocation entry point checks everything on the host before
    its first HIP call: partials larger than the fixed device array are
    refused with PKV_ERR_WORKSPACE, other argument errors as usual."""
    L = _lib.lib()

    def call(B=64, Hq=16, Hkv=8, max_len=4096, out=FAKE, kn=FAKE, split=0):
        return L.pkv_paged_decode_attention_store_noalloc(out, 0, FAKE, 0, FAKE, FAKE, kn, FAKE, 0,
                                                          FAKE, 16, FAKE, B, Hq, Hkv, 128, 256,
                                                          600, max_len, 0.0, split, None)

    big = L.pkv_decode_workspace_bytes(64, 64, 8, 128, 131072, 0)
    assert big > _lib.PKV_STATIC_SCRATCH_BYTES
    assert call(Hq=64, max_len=131072) == _lib.PKV_ERR_WORKSPACE
    assert b"fixed" in L.pkv_last_error()
    assert call(out=None) == _lib.PKV_ERR_INVALID_ARG
    assert call(kn=FAKE + 2) == _lib.PKV_ERR_INVALID_ARG
    assert call(split=100) == _lib.PKV_ERR_INVALID_ARG
    assert call(B=0) == _lib.PKV_OK     # nothing to do, no HIP call


def test_cascade_validation():
    L = _lib.lib()
    need = L.pkv_cascade_workspace_bytes(16, 10, 10, 128, 1281, 4, 256, 0)
    assert need > 0
    # more than the plain split-KV workspace of the same batch: prefix partials come first
    assert need >= L.pkv_decode_workspace_bytes(16, 10, 10, 128, 1281 - 1024, 0)
    assert L.pkv_cascade_workspace_bytes(16, 10, 10, 128, 1281, 0, 256, 0) == 0
    assert L.pkv_cascade_workspace_bytes(16, 12, 8, 128, 1281, 4, 256, 0) == 0
    assert L.pkv_cascade_workspace_bytes(16, 10, 10, 128, 1281, 4, 256, 100) == 0

    def call(**kw):
        a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, pb=FAKE, npb=4, bt=FAKE, lens=FAKE, D=128,
                 ws=FAKE, wsb=need)
        a.update(kw)
        return L.pkv_cascade_decode_attention(a["out"], 0, a["q"], 0, a["k"], a["v"], a["pb"],
                                              a["npb"], a["bt"], 6, a["lens"], 16, 10, 10, a["D"],
                                              256, 40, 1281, 0.0, 0, a["ws"], a["wsb"], None)

    assert call(pb=None) == _lib.PKV_ERR_INVALID_ARG
    assert call(pb=FAKE + 2) == _lib.PKV_ERR_INVALID_ARG
    assert call(npb=0) == _lib.PKV_ERR_INVALID_ARG
    assert call(out=None) == _lib.PKV_ERR_INVALID_ARG
    assert call(q=None) == _lib.PKV_ERR_INVALID_ARG
    assert call(D=96) == _lib.PKV_ERR_UNSUPPORTED
    assert call(ws=None) == _lib.PKV_ERR_WORKSPACE
    assert call(wsb=need - 1) == _lib.PKV_ERR_WORKSPACE


def test_sampler_ex_validation():
    L = _lib.lib()
    need = L.pkv_sampler_workspace_bytes(4, 1000)

    def call(**kw):
        a = dict(ids=FAKE, z=FAKE, g=FAKE, m=None, ms=0, t=FAKE, p=FAKE, k=FAKE, B=4, V=1000,
                 prob=None, tid=None, tpr=None, ws=FAKE, wsb=need)
        a.update(kw)
        return L.pkv_sample_next_token_ex(a["ids"], a["z"], 0, a["g"], 0, a["m"], a["ms"], a["t"],
                                          a["p"], a["k"], a["B"], a["V"], a["prob"], a["tid"],
                                          a["tpr"], a["ws"], a["wsb"], None)

    assert call(m=FAKE, ms=999) == _lib.PKV_ERR_INVALID_ARG     # mask stride below vocab
    assert call(prob=FAKE + 2) == _lib.PKV_ERR_INVALID_ARG      # misaligned output
    assert call(tid=FAKE + 1) == _lib.PKV_ERR_INVALID_ARG
    assert call(z=None) == _lib.PKV_ERR_INVALID_ARG
    assert call(wsb=need - 1) == _lib.PKV_ERR_WORKSPACE
    assert call(B=0, ids=None, z=None, g=None, t=None, p=None, k=None) == _lib.PKV_OK


def test_varlen_validation():
    L = _lib.lib()

    # one sequence, 512 new tokens after a long prefix: 64 row tiles, so the
    # automatic choice splits each causal range in 4
    need = L.pkv_varlen_workspace_bytes(512, 1, 16, 8, 128, 512, 65536, 0)

    def call(**kw):
        a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, cq=FAKE, ck=FAKE, B=1, T=512, Hq=16,
                 Hkv=8, D=128, bs=256, mq=512, mk=65536, qs=0, scale=0.0, split=0, ws=FAKE,
                 wsb=need)
        a.update(kw)
        return L.pkv_varlen_paged_attention(a["out"], 0, a["q"], a["qs"], a["k"], a["v"], a["bt"],
                                            256, a["cq"], a["ck"], a["B"], a["T"], a["Hq"],
                                            a["Hkv"], a["D"], a["bs"], 600, a["mq"], a["mk"],
                                            a["scale"], a["split"], a["ws"], a["wsb"], None)

    # automatic split: only up to about one workgroup per CU, >= 1024
    # positions, never longer than the longest range needs (then no workspace)
    assert L.pkv_varlen_split_tokens(1, 16, 8, 512, 65536, 0) == 16384
    assert L.pkv_varlen_split_tokens(4, 16, 8, 512, 2048, 0) == 2048
    assert L.pkv_varlen_split_tokens(2, 16, 8, 512, 8192, 0) == 4096
    assert L.pkv_varlen_split_tokens(7, 4, 2, 64, 364, 0) == 512
    assert L.pkv_varlen_split_tokens(4, 16, 8, 512, 4096, 512) == 512
    assert L.pkv_varlen_split_tokens(4, 16, 8, 512, 4096, 100) == 0
    assert need == (512 * 16 * 4 * 128 * 4) + (512 * 16 * 4 * 2 * 4)
    assert L.pkv_varlen_workspace_bytes(2048, 4, 16, 8, 128, 512, 2048, 0) == 0
    assert L.pkv_varlen_workspace_bytes(7, 7, 4, 2, 128, 64, 364, 0) == 0
    assert call(ws=None) == _lib.PKV_ERR_WORKSPACE
    assert call(wsb=need - 1) == _lib.PKV_ERR_WORKSPACE
    assert call(ws=FAKE + 16) == _lib.PKV_ERR_WORKSPACE
    assert call(split=100) == _lib.PKV_ERR_INVALID_ARG
    assert call(T=-1) == _lib.PKV_ERR_INVALID_ARG
    assert call(T=0, out=None, q=None) == _lib.PKV_OK
    assert call(cq=None) == _lib.PKV_ERR_INVALID_ARG
    assert call(out=FAKE + 8) == _lib.PKV_ERR_INVALID_ARG
    assert call(D=96) == _lib.PKV_ERR_UNSUPPORTED
    assert call(Hq=12) == _lib.PKV_ERR_INVALID_ARG
    assert call(qs=16 * 128 - 8) == _lib.PKV_ERR_INVALID_ARG
    assert call(mq=-1) == _lib.PKV_ERR_INVALID_ARG
    assert call(scale=float("inf")) == _lib.PKV_ERR_INVALID_ARG
    assert call(mq=0, out=None, q=None) == _lib.PKV_OK
    assert L.pkv_varlen_slot_mapping(None, FAKE, 4, FAKE, FAKE, 3, 10, 16, None) == \
        _lib.PKV_ERR_INVALID_ARG
    assert L.pkv_varlen_slot_mapping(FAKE, FAKE, 4, FAKE, FAKE, 3, 10, 24, None) == \
        _lib.PKV_ERR_UNSUPPORTED
    assert L.pkv_varlen_slot_mapping(None, None, 4, None, None, 0, 10, 16, None) == _lib.PKV_OK
