"""GPU parity of varlen multi-query paged attention (chunked prefill over a
paged cache with a cached prefix) and of its slot mapping, against the CPU
oracle.  Bars: slots and stored pools bit-exact; attention within max-abs
1e-2 of the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_store_amd as pkv
from workloads.generate import bf16_bits_from_f32

from gpu_util import ATTN_TOL, bf16_out_to_f64, dev_i32, dev_u16, host_u16, oracle_head_jobs, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _normal_bf16(rng, shape):
    return bf16_bits_from_f32(rng.standard_normal(size=shape, dtype=np.float32))


def _case(rng, lens_cached, lens_new, Hq, Hkv, D, bs, spare=3):
    """A fragmented pool holding each sequence's cached tokens (every other
    pool byte random), the new tokens' q/k/v, and the varlen arguments."""
    B = len(lens_new)
    total = [c + n for c, n in zip(lens_cached, lens_new)]
    need = [max(1, (t + bs - 1) // bs) for t in total]
    nb = sum(need) + spare
    perm = rng.permutation(nb).astype(np.int32)
    W = max(need)
    tables = np.full((B, W), -1, np.int32)
    pos = 0
    for b in range(B):
        tables[b, :need[b]] = perm[pos:pos + need[b]]
        pos += need[b]
    kp, vp = _normal_bf16(rng, (nb, bs, Hkv, D)), _normal_bf16(rng, (nb, bs, Hkv, D))
    T = int(sum(lens_new))
    q = _normal_bf16(rng, (T, Hq, D))
    kn, vn = _normal_bf16(rng, (T, Hkv, D)), _normal_bf16(rng, (T, Hkv, D))
    cu_q = np.concatenate([[0], np.cumsum(lens_new)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(total)]).astype(np.int32)
    return q, kp, vp, kn, vn, tables, cu_q, cu_k


def _prefill(q, kp, vp, kn, vn, tables, cu_q, cu_k, bs, split=0):
    """GPU: slots of the new tokens, store, varlen attention (split_tokens
    `split`: 0 automatic, else positions per split of a tile's range)."""
    lens_new = np.diff(cu_q)
    lens_k = np.diff(cu_k)
    mq, mk = int(lens_new.max()), int(lens_k.max())
    kc, vc = dev_u16(kp), dev_u16(vp)
    td, cq, ck = dev_i32(tables), dev_i32(cu_q), dev_i32(cu_k)
    slots = pkv.varlen_slot_mapping(td, cq, ck, mq, bs, int(cu_q[-1]))
    pkv.kv_store(kc, vc, dev_u16(kn), dev_u16(vn), slots)
    out = pkv.varlen_paged_attention(dev_u16(q), kc, vc, td, cq, ck, mq, mk, split_tokens=split)
    torch.cuda.synchronize()
    return slots.cpu().numpy(), host_u16(kc), host_u16(vc), bf16_out_to_f64(out)


def _reference(q, kp, vp, kn, vn, tables, cu_q, cu_k, bs, rows=None):
    s_ref = oracle.varlen_slot_mapping(tables, cu_q, cu_k, bs)
    kref, vref = kp.copy(), vp.copy()
    assert oracle.kv_store(kref, vref, kn, vn, s_ref, bs) == 0
    if rows is None:
        return s_ref, kref, vref, oracle.varlen_attention(q, kref, vref, tables, cu_q, cu_k)
    return s_ref, kref, vref, None


# Block sizes below the 64-position tile (128 at head_dim 64) take the
# per-position block-id path, the others one block id per tile; 64 at head_dim
# 128 and 128 at head_dim 64 are the boundary cases.
@pytest.mark.parametrize("D,Hq,Hkv,bs", [(128, 4, 2, 16), (64, 6, 2, 32), (128, 8, 8, 256),
                                         (128, 16, 1, 16), (64, 12, 4, 64), (128, 9, 3, 16),
                                         (128, 6, 2, 64), (64, 8, 2, 128), (64, 4, 4, 256),
                                         (128, 48, 8, 256)])
@pytest.mark.parametrize("split", [0, 256])
def test_varlen_matches_oracle(D, Hq, Hkv, bs, split):
    """split 256: ranges longer than 256 positions go through partials and
    the log-sum-exp merge (the automatic choice keeps these in one split)."""
    rng = np.random.default_rng(D + 7 * Hq + 3 * Hkv + bs)
    lens_cached = [0, 5, 40, 0, 300, 17, 64]
    lens_new = [1, 33, 7, 50, 2, 64, 1]
    args = _case(rng, lens_cached, lens_new, Hq, Hkv, D, bs)
    say(f"varlen D={D} Hq={Hq} Hkv={Hkv} bs={bs} split={split} cached={lens_cached} new={lens_new}")
    slots, kc, vc, got = _prefill(*args, bs, split)
    s_ref, kref, vref, ref = _reference(*args, bs)
    assert np.array_equal(slots, s_ref)
    assert np.array_equal(kc, kref) and np.array_equal(vc, vref)
    err = np.abs(got - ref).max()
    say(f"  max abs err {err:.3e}")
    assert err <= ATTN_TOL


@pytest.mark.parametrize("split", [0, 512])
def test_varlen_empty_sequence_and_long_prefix(split):
    """A sequence with no new tokens between others (its rows do not exist,
    the rest are unaffected), a prefix spanning many tiles with a chunk that
    ends inside a tile, and a chunk longer than one 128-row tile."""
    rng = np.random.default_rng(77)
    lens_cached = [10, 20, 0, 1500, 129]
    lens_new = [3, 0, 70, 37, 200]
    args = _case(rng, lens_cached, lens_new, 8, 4, 128, 256)
    say(f"varlen empty/long split={split} cached={lens_cached} new={lens_new}")
    slots, kc, vc, got = _prefill(*args, 256, split)
    s_ref, kref, vref, ref = _reference(*args, 256)
    assert np.array_equal(slots, s_ref)
    assert np.array_equal(kc, kref) and np.array_equal(vc, vref)
    err = np.abs(got - ref).max()
    say(f"  max abs err {err:.3e}")
    assert err <= ATTN_TOL


def test_varlen_long_prefix_automatic_split():
    """One sequence, 100 new tokens after a 6000-token cached prefix: only 8
    row tiles, so the automatic choice splits the causal range (6 splits of
    1024 positions) and merges."""
    rng = np.random.default_rng(91)
    lens_cached, lens_new = [6000], [100]
    Hq, Hkv, D, bs = 8, 2, 128, 256
    assert pkv.varlen_split_tokens(1, Hq, Hkv, 100, 6100) == 1024
    args = _case(rng, lens_cached, lens_new, Hq, Hkv, D, bs)
    say("varlen long prefix, automatic split")
    slots, kc, vc, got = _prefill(*args, bs)
    s_ref, kref, vref, ref = _reference(*args, bs)
    assert np.array_equal(slots, s_ref)
    err = np.abs(got - ref).max()
    say(f"  max abs err {err:.3e}")
    assert err <= ATTN_TOL


def test_varlen_one_new_token_equals_decode():
    """q_len = 1 for every sequence: the decode step's attention."""
    rng = np.random.default_rng(31)
    lens_cached = [16, 0, 250, 511, 3]
    args = _case(rng, lens_cached, [1] * 5, 16, 8, 128, 256)
    q, kp, vp, kn, vn, tables, cu_q, cu_k = args
    slots, kc, vc, got = _prefill(*args, 256)
    lens = np.diff(cu_k).astype(np.int32)
    kd, vd = dev_u16(kc), dev_u16(vc)
    dec = pkv.paged_decode_attention(dev_u16(q), kd, vd, dev_i32(tables), dev_i32(lens),
                                     int(lens.max()))
    torch.cuda.synchronize()
    assert np.abs(got - bf16_out_to_f64(dec)).max() <= ATTN_TOL
    s_ref, kref, vref, ref = _reference(*args, 256)
    assert np.abs(got - ref).max() <= ATTN_TOL


def test_varlen_qwen3_shaped_chunk_every_output():
    """A Qwen3-shaped chunked-prefill batch (GQA 16/8, D 128, block 256):
    4 sequences of 512 new tokens after cached prefixes of 0..1536 tokens;
    every one of the 2048 x 16 (token, head) outputs against the threaded
    oracle."""
    rng = np.random.default_rng(32)
    Hq, Hkv, D, bs = 16, 8, 128, 256
    lens_cached, lens_new = [0, 256, 1024, 1536], [512] * 4
    args = _case(rng, lens_cached, lens_new, Hq, Hkv, D, bs)
    q, kp, vp, kn, vn, tables, cu_q, cu_k = args
    say("varlen qwen3-shaped chunk")
    slots, kc, vc, got = _prefill(*args, bs)
    s_ref, kref, vref, _ = _reference(*args, bs, rows=True)
    assert np.array_equal(slots, s_ref)
    assert np.array_equal(kc, kref) and np.array_equal(vc, vref)
    g = Hq // Hkv
    jobs = []
    for b in range(4):
        for j in range(lens_new[b]):
            row = int(cu_q[b]) + j
            jobs += [((row, h), q[row, h], tables[b], lens_cached[b] + j + 1, h // g)
                     for h in range(Hq)]
    ref = oracle_head_jobs(jobs, kref, vref, 1.0 / np.sqrt(D))
    worst = max(float(np.abs(got[r, h] - ref[(r, h)]).max()) for r, h in ref)
    say(f"  max abs err over all {len(ref)} outputs {worst:.3e}")
    assert worst <= ATTN_TOL