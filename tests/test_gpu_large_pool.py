"""GPU: KV pools whose element offsets pass 2^31 (8,400 blocks of 256
positions x 8 KV heads x 128 dims: 2.2 G bf16 elements, 4.4 GB per pool).
Rows reference blocks on both sides of the 2^31-element mark; the slot
mapping and store, the fused store, and both partial kernels (group 2 on
the VALU kernel, group 6 on the matrix cores) must address them with
64-bit offsets.  Only the referenced blocks are written (the rest of each
pool is left uninitialised and never read) and only those are copied back:
the oracle sees a compact pool with the block tables renumbered."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_store_amd as pkv
from workloads.generate import bf16_bits_from_f32

from gpu_util import ATTN_TOL, bf16_out_to_f64, dev_i32, dev_u16, host_u16, say

pytestmark = pytest.mark.gpu

NB, BS, HKV, D = 8400, 256, 8, 128   # 2^31 elements = 8192 blocks


@pytest.fixture(scope="module")
def pools():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    assert NB * BS * HKV * D > 2 ** 31
    kc = torch.empty((NB, BS, HKV, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    yield kc, vc
    del kc, vc
    torch.cuda.empty_cache()


def _normal_bf16(rng, shape):
    return bf16_bits_from_f32(rng.standard_normal(size=shape, dtype=np.float32))


def _setup(rng, kc, vc, lens):
    """Block tables over both sides of the 2^31-element mark; the
    referenced blocks get seeded values on the device and are returned as a
    compact host pool with renumbered tables."""
    need = [max(1, -(-n // BS)) for n in lens]
    high = rng.permutation(np.arange(8150, NB))          # around and past block 8192
    low = rng.permutation(np.arange(0, 300))
    ids, hi_i, lo_i = [], 0, 0
    for k in need:
        row = []
        for j in range(k):
            if j % 3 == 2:
                row.append(int(low[lo_i])); lo_i += 1
            else:
                row.append(int(high[hi_i])); hi_i += 1
        ids.append(row)
    tables = np.full((len(lens), max(need)), -1, np.int32)
    for b, row in enumerate(ids):
        tables[b, :len(row)] = row
    used = np.array(sorted({x for row in ids for x in row}), np.int64)
    kblk, vblk = _normal_bf16(rng, (len(used), BS, HKV, D)), _normal_bf16(rng, (len(used), BS, HKV, D))
    idx = torch.from_numpy(used).cuda()
    kc.view(torch.int16).index_copy_(0, idx, torch.from_numpy(kblk.view(np.int16)).cuda())
    vc.view(torch.int16).index_copy_(0, idx, torch.from_numpy(vblk.view(np.int16)).cuda())
    remap = {int(x): i for i, x in enumerate(used)}
    compact = np.full_like(tables, -1)
    for b, row in enumerate(ids):
        compact[b, :len(row)] = [remap[x] for x in row]
    return tables, compact, used


def _host_blocks(pool, used):
    return host_u16(pool.index_select(0, torch.from_numpy(used).cuda()))


@pytest.mark.parametrize("Hq", [16, 48])
def test_attention_over_blocks_past_2_31_elements(pools, Hq):
    kc, vc = pools
    rng = np.random.default_rng(3000 + Hq)
    lens = [300, 5000, 1, 777, 2600]
    tables, compact, used = _setup(rng, kc, vc, lens)
    assert int(tables.max()) * BS * HKV * D > 2 ** 31
    n = np.asarray(lens, np.int32)
    q = _normal_bf16(rng, (len(lens), Hq, D))
    say(f"large pool Hq={Hq}: blocks up to {tables.max()}")
    got = pkv.paged_decode_attention(dev_u16(q), kc, vc, dev_i32(tables), dev_i32(n), int(n.max()))
    torch.cuda.synchronize()
    ref = oracle.decode_attention(q, _host_blocks(kc, used), _host_blocks(vc, used), compact, n)
    err = float(np.abs(bf16_out_to_f64(got) - ref).max())
    say(f"  max abs err {err:.3e}")
    assert err <= ATTN_TOL


def test_store_and_fused_store_past_2_31_elements(pools):
    kc, vc = pools
    rng = np.random.default_rng(3100)
    lens = [257, 4000, 513, 1]
    tables, compact, used = _setup(rng, kc, vc, lens)
    n = np.asarray(lens, np.int32)
    B = len(lens)
    td, nd = dev_i32(tables), dev_i32(n)
    # slot mapping + store: the new rows land at slot(context_len - 1)
    kn, vn = _normal_bf16(rng, (B, HKV, D)), _normal_bf16(rng, (B, HKV, D))
    slots = pkv.slot_mapping(td, nd, BS)
    torch.cuda.synchronize()
    s_host = slots.cpu().numpy()
    assert np.array_equal(s_host, oracle.slot_mapping(tables, n, BS))
    assert (s_host.astype(np.int64) * HKV * D).max() > 2 ** 31
    pkv.kv_store(kc, vc, dev_u16(kn), dev_u16(vn), slots)
    torch.cuda.synchronize()
    kh, vh = host_u16(kc.view(NB * BS, HKV, D)[slots.long()]), host_u16(vc.view(NB * BS, HKV, D)[slots.long()])
    assert np.array_equal(kh, kn) and np.array_equal(vh, vn)

    # fused store + attention with new rows again; then compare with the oracle
    kn2, vn2 = _normal_bf16(rng, (B, HKV, D)), _normal_bf16(rng, (B, HKV, D))
    Hq = 16
    q = _normal_bf16(rng, (B, Hq, D))
    got = pkv.paged_decode_attention_store(dev_u16(q), kc, vc, dev_u16(kn2), dev_u16(vn2), td, nd,
                                           int(n.max()))
    torch.cuda.synchronize()
    kh, vh = host_u16(kc.view(NB * BS, HKV, D)[slots.long()]), host_u16(vc.view(NB * BS, HKV, D)[slots.long()])
    assert np.array_equal(kh, kn2) and np.array_equal(vh, vn2)
    ref = oracle.decode_attention(q, _host_blocks(kc, used), _host_blocks(vc, used), compact, n)
    err = float(np.abs(bf16_out_to_f64(got) - ref).max())
    say(f"  fused store: max abs err {err:.3e}")
    assert err <= ATTN_TOL
