"""GPU: the device error word.

Contract violations in device-side contents (a slot past the pool, a block
id outside [0, num_blocks), a length past max_context_len or the table,
inconsistent varlen lengths, a bounded wait that gives up) set their
PKV_DEVERR_* bit in the caller's word while every kernel stays inside its
buffers; valid rows keep their exact results.  Nothing here faults: bad ids
are clamped by the kernels, and the bounded wait is made to give up by a
host-side poll cap, not by breaking the kernel.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_store_amd as pkv
from workloads.generate import bf16_bits_from_f32

from gpu_util import ATTN_TOL, bf16_out_to_f64, dev_i32, dev_u16, host_u16, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


@pytest.fixture()
def word():
    w = torch.zeros(1, dtype=torch.int32, device="cuda")
    pkv.set_error_word(w)
    yield w
    pkv.set_error_word(None)
    pkv.set_wait_limit(0)


def _bits(w):
    torch.cuda.synchronize()
    return int(w.item()) & 0xffffffff


def _bf16(rng, shape):
    return bf16_bits_from_f32(rng.standard_normal(size=shape, dtype=np.float32))


def _paged(rng, n, Hq, Hkv, D, bs, spare=2):
    B = len(n)
    need = [max(1, (x + bs - 1) // bs) for x in n]
    nb = sum(need) + spare
    perm = rng.permutation(nb).astype(np.int32)
    W = max(need)
    t = np.zeros((B, W), np.int32)
    pos = 0
    for b in range(B):
        t[b, :need[b]] = perm[pos:pos + need[b]]
        pos += need[b]
    return t, nb, _bf16(rng, (nb, bs, Hkv, D)), _bf16(rng, (nb, bs, Hkv, D)), _bf16(rng, (B, Hq, D))


def test_valid_inputs_leave_the_word_clear(word):
    rng = np.random.default_rng(1)
    n = np.array([1, 77, 300, 0], np.int32)
    for Hq, Hkv in ((8, 4), (12, 2)):   # VALU and matrix-core partial kernels
        t, nb, kp, vp, q = _paged(rng, n, Hq, Hkv, 128, 16)
        kc, vc = dev_u16(kp), dev_u16(vp)
        slots = pkv.slot_mapping(dev_i32(t), dev_i32(n), 16)
        pkv.kv_store(kc, vc, dev_u16(_bf16(rng, (4, Hkv, 128))), dev_u16(_bf16(rng, (4, Hkv, 128))),
                     slots)
        pkv.paged_decode_attention(dev_u16(q), kc, vc, dev_i32(t), dev_i32(n), 300, split_tokens=64)
        assert _bits(word) == 0


def test_store_slot_past_the_pool(word):
    rng = np.random.default_rng(2)
    nb, bs, hkv, d = 6, 16, 2, 64
    kp, vp = _bf16(rng, (nb, bs, hkv, d)), _bf16(rng, (nb, bs, hkv, d))
    kn, vn = _bf16(rng, (3, hkv, d)), _bf16(rng, (3, hkv, d))
    slots = np.array([5, nb * bs, 40], np.int32)    # the middle one is past the pool
    kc, vc = dev_u16(kp), dev_u16(vp)
    pkv.kv_store(kc, vc, dev_u16(kn), dev_u16(vn), dev_i32(slots))
    assert _bits(word) == pkv.PKV_DEVERR_SLOT
    kref, vref = kp.copy(), vp.copy()
    ok = slots.copy()
    ok[1] = -1
    assert oracle.kv_store(kref, vref, kn, vn, ok, bs) == 0
    assert np.array_equal(host_u16(kc), kref) and np.array_equal(host_u16(vc), vref)


def test_slot_mapping_missing_block_and_short_table(word):
    t = np.array([[5, -1], [3, 4]], np.int32)
    n = np.array([20, 2], np.int32)          # row 0's position 19 needs the -1 entry
    got = pkv.slot_mapping(dev_i32(t), dev_i32(n), 16).cpu().numpy()
    assert _bits(word) == pkv.PKV_DEVERR_BLOCK_ID
    assert got.tolist() == oracle.slot_mapping(t, n, 16).tolist()
    word.zero_()
    n2 = np.array([40, 2], np.int32)         # past the two-entry table
    pkv.slot_mapping(dev_i32(t), dev_i32(n2), 16)
    assert _bits(word) == pkv.PKV_DEVERR_CONTEXT_LEN


@pytest.mark.parametrize("Hq,Hkv", [(8, 4), (16, 2)], ids=["valu", "mfma"])
def test_attention_bad_block_ids_and_lengths(word, Hq, Hkv):
    rng = np.random.default_rng(3)
    D, bs = 128, 16
    n = np.array([50, 90, 33], np.int32)
    t, nb, kp, vp, q = _paged(rng, n, Hq, Hkv, D, bs)
    ref = oracle.decode_attention(q, kp, vp, t, n)
    bad = t.copy()
    bad[1, 2] = -7          # row 1: two bad ids inside its context
    bad[1, 4] = nb + 3
    out = pkv.paged_decode_attention(dev_u16(q), dev_u16(kp), dev_u16(vp), dev_i32(bad),
                                     dev_i32(n), 96, split_tokens=64)
    assert _bits(word) == pkv.PKV_DEVERR_BLOCK_ID
    got = bf16_out_to_f64(out)
    for b in (0, 2):        # the other rows are unaffected
        assert np.abs(got[b] - ref[b]).max() <= ATTN_TOL
    # a length past max_context_len is truncated and reported
    word.zero_()
    n2 = n.copy()
    n2[2] = 200
    pkv.paged_decode_attention(dev_u16(q), dev_u16(kp), dev_u16(vp), dev_i32(t), dev_i32(n2), 96,
                               split_tokens=64)
    assert _bits(word) == pkv.PKV_DEVERR_CONTEXT_LEN


def test_fused_store_with_a_bad_block_id(word):
    rng = np.random.default_rng(4)
    D, bs, Hq, Hkv = 64, 16, 4, 2
    n = np.array([40, 17], np.int32)
    t, nb, kp, vp, q = _paged(rng, n, Hq, Hkv, D, bs)
    bad = t.copy()
    bad[0, 2] = nb           # the block of row 0's new position 39
    kn, vn = _bf16(rng, (2, Hkv, D)), _bf16(rng, (2, Hkv, D))
    kc, vc = dev_u16(kp), dev_u16(vp)
    pkv.paged_decode_attention_store(dev_u16(q), kc, vc, dev_u16(kn), dev_u16(vn), dev_i32(bad),
                                     dev_i32(n), 64)
    assert _bits(word) == pkv.PKV_DEVERR_BLOCK_ID
    # row 1's new token was stored; row 0's was skipped (its block is invalid)
    kref, vref = kp.copy(), vp.copy()
    s = oracle.slot_mapping(bad, n, bs)
    s[0] = -1
    assert oracle.kv_store(kref, vref, kn, vn, s, bs) == 0
    assert np.array_equal(host_u16(kc), kref) and np.array_equal(host_u16(vc), vref)


def _varlen_case(rng, cached, new, Hq=8, Hkv=4, D=128, bs=16):
    total = [c + x for c, x in zip(cached, new)]
    need = [(x + bs - 1) // bs for x in total]
    nb = sum(need) + 2
    perm = rng.permutation(nb).astype(np.int32)
    t = np.zeros((len(new), max(need)), np.int32)
    pos = 0
    for b, k in enumerate(need):
        t[b, :k] = perm[pos:pos + k]
        pos += k
    q = _bf16(rng, (sum(new), Hq, D))
    cu_q = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(total)]).astype(np.int32)
    return q, _bf16(rng, (nb, bs, Hkv, D)), _bf16(rng, (nb, bs, Hkv, D)), t, cu_q, cu_k


def test_varlen_bad_block_and_lengths(word):
    rng = np.random.default_rng(5)
    q, kp, vp, t, cu_q, cu_k = _varlen_case(rng, (100, 30), (64, 40))
    ref = oracle.varlen_attention(q, kp, vp, t, cu_q, cu_k)
    bad = t.copy()
    bad[1, 1] = -2
    out = pkv.varlen_paged_attention(dev_u16(q), dev_u16(kp), dev_u16(vp), dev_i32(bad),
                                     dev_i32(cu_q), dev_i32(cu_k), 64, 164)
    assert _bits(word) == pkv.PKV_DEVERR_BLOCK_ID
    got = bf16_out_to_f64(out)
    assert np.abs(got[:64] - ref[:64]).max() <= ATTN_TOL     # sequence 0 is unaffected
    # k_len < q_len for sequence 1: it writes nothing and is reported
    word.zero_()
    cu_k2 = cu_k.copy()
    cu_k2[2] = cu_k2[1] + 10
    pkv.varlen_paged_attention(dev_u16(q), dev_u16(kp), dev_u16(vp), dev_i32(t), dev_i32(cu_q),
                               dev_i32(cu_k2), 64, 164)
    assert _bits(word) == pkv.PKV_DEVERR_SEQLENS


def test_varlen_wait_that_gives_up_is_reported(word):
    """With a one-poll cap the per-group step synchronisation gives up while
    other waves are still staging; the launch still ends normally (every
    address is independent of the wait) and reports PKV_DEVERR_WAIT.  With
    the default cap restored the same call is correct and reports nothing."""
    rng = np.random.default_rng(6)
    q, kp, vp, t, cu_q, cu_k = _varlen_case(rng, (1500, 900), (256, 256), bs=256)
    args = (dev_u16(q), dev_u16(kp), dev_u16(vp), dev_i32(t), dev_i32(cu_q), dev_i32(cu_k), 256,
            1756)
    pkv.set_wait_limit(1)
    say("varlen with a one-poll wait cap")
    pkv.varlen_paged_attention(*args)
    assert _bits(word) & pkv.PKV_DEVERR_WAIT
    pkv.set_wait_limit(0)
    word.zero_()
    out = pkv.varlen_paged_attention(*args)
    assert _bits(word) == 0
    ref = oracle.varlen_attention(q, kp, vp, t, cu_q, cu_k)
    assert np.abs(bf16_out_to_f64(out) - ref).max() <= ATTN_TOL


def test_no_word_means_no_reporting():
    """The default: no word set, bad ids still stay in bounds."""
    pkv.set_error_word(None)
    rng = np.random.default_rng(7)
    n = np.array([40], np.int32)
    t, nb, kp, vp, q = _paged(rng, n, 4, 2, 64, 16)
    t[0, 0] = 1 << 30
    pkv.paged_decode_attention(dev_u16(q), dev_u16(kp), dev_u16(vp), dev_i32(t), dev_i32(n), 64)
    torch.cuda.synchronize()
