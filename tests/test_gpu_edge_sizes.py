"""GPU: size limits of the decode path.  The largest block size (4096
positions per block) with rows ending just before, at and after block
boundaries, on both partial kernels and with the fused store; and a large
batch (2,048 rows of ragged short contexts, empty rows included) for the
slot mapping, the store and attention.  Slots and pools bit-exact, outputs
within the attention bar of the fp64 oracle."""
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


def _normal_bf16(rng, shape):
    return bf16_bits_from_f32(rng.standard_normal(size=shape, dtype=np.float32))


def _case(rng, lens, Hkv, D, bs):
    need = [max(1, -(-n // bs)) for n in lens]
    nb = sum(need) + 1
    perm = rng.permutation(nb).astype(np.int32)
    tables = np.full((len(lens), max(need)), -1, np.int32)
    pos = 0
    for b, k in enumerate(need):
        tables[b, :k] = perm[pos:pos + k]
        pos += k
    kp, vp = _normal_bf16(rng, (nb, bs, Hkv, D)), _normal_bf16(rng, (nb, bs, Hkv, D))
    return kp, vp, tables, np.asarray(lens, np.int32)


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 8, 8), (128, 16, 8), (128, 48, 8), (64, 12, 4)])
def test_block_size_4096(D, Hq, Hkv):
    bs = 4096
    rng = np.random.default_rng(4000 + D + Hq)
    lens = [1, 4095, 4096, 4097, 9000, 0, 8192]
    kp, vp, tables, n = _case(rng, lens, Hkv, D, bs)
    B, max_len = len(lens), int(n.max())
    q = _normal_bf16(rng, (B, Hq, D))
    kn, vn = _normal_bf16(rng, (B, Hkv, D)), _normal_bf16(rng, (B, Hkv, D))
    say(f"block 4096 D={D} Hq={Hq} Hkv={Hkv}")
    td, nd = dev_i32(tables), dev_i32(n)
    slots = pkv.slot_mapping(td, nd, bs)
    torch.cuda.synchronize()
    s_host = slots.cpu().numpy()
    assert np.array_equal(s_host, oracle.slot_mapping(tables, n, bs))

    kc, vc = dev_u16(kp), dev_u16(vp)
    got = pkv.paged_decode_attention_store(dev_u16(q), kc, vc, dev_u16(kn), dev_u16(vn), td, nd,
                                           max_len)
    torch.cuda.synchronize()
    # the pools after the store: the oracle's store into copies of the host pools
    kref, vref = kp.copy(), vp.copy()
    live = n >= 1
    oracle.kv_store(kref, vref, kn[live], vn[live], s_host[live], bs)
    assert np.array_equal(host_u16(kc), kref) and np.array_equal(host_u16(vc), vref)
    ref = oracle.decode_attention(q, kref, vref, tables, n)
    out = bf16_out_to_f64(got)
    assert not out[5].any(), "an empty row's output is the zero vector"
    err = float(np.abs(out - ref).max())
    say(f"  max abs err {err:.3e}")
    assert err <= ATTN_TOL


def test_large_batch_ragged_short_rows():
    B, Hq, Hkv, D, bs = 2048, 16, 8, 128, 16
    rng = np.random.default_rng(4100)
    lens = rng.integers(0, 301, B)
    lens[::97] = 0
    kp, vp, tables, n = _case(rng, lens, Hkv, D, bs)
    q = _normal_bf16(rng, (B, Hq, D))
    kn, vn = _normal_bf16(rng, (B, Hkv, D)), _normal_bf16(rng, (B, Hkv, D))
    say(f"large batch B={B}, blocks {kp.shape[0]}")
    td, nd = dev_i32(tables), dev_i32(n)
    slots = pkv.slot_mapping(td, nd, bs)
    torch.cuda.synchronize()
    s_host = slots.cpu().numpy()
    assert np.array_equal(s_host, oracle.slot_mapping(tables, n, bs))
    kc, vc = dev_u16(kp), dev_u16(vp)
    live = n >= 1
    pkv.kv_store(kc, vc, dev_u16(kn[live]), dev_u16(vn[live]), slots[torch.from_numpy(live).cuda()])
    torch.cuda.synchronize()
    kref, vref = kp.copy(), vp.copy()
    oracle.kv_store(kref, vref, kn[live], vn[live], s_host[live], bs)
    assert np.array_equal(host_u16(kc), kref) and np.array_equal(host_u16(vc), vref)
    got = pkv.paged_decode_attention(dev_u16(q), kc, vc, td, nd, int(n.max()))
    torch.cuda.synchronize()
    ref = oracle.decode_attention(q, kref, vref, tables, n)
    out = bf16_out_to_f64(got)
    assert not out[0].any()
    err = float(np.abs(out - ref).max())
    say(f"  max abs err {err:.3e}")
    assert err <= ATTN_TOL
