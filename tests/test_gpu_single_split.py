"""GPU: decode attention when every row fits in one split.  The combined
entry points then skip the reduce step and the partial kernel writes the
normalised output itself; that output must equal the two-step path with the
same split bit for bit, stay within the attention bar of the fp64 oracle,
and be the zero vector for empty rows.  Covers both partial kernels (group
sizes 1 and 2 on the VALU kernel, 6 and 1x10 on the matrix-core kernel),
head_dim 64/128, several block sizes, and the fused store variant."""
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


def _case(rng, lens, Hq, Hkv, D, bs, spare=2):
    need = [max(1, (n + bs - 1) // bs) for n in lens]
    nb = sum(need) + spare
    perm = rng.permutation(nb).astype(np.int32)
    tables = np.full((len(lens), max(need)), -1, np.int32)
    pos = 0
    for b, k in enumerate(need):
        tables[b, :k] = perm[pos:pos + k]
        pos += k
    kp, vp = _normal_bf16(rng, (nb, bs, Hkv, D)), _normal_bf16(rng, (nb, bs, Hkv, D))
    q = _normal_bf16(rng, (len(lens), Hq, D))
    return q, kp, vp, tables, np.asarray(lens, np.int32)


SHAPES = [(128, 16, 8, 256), (64, 16, 16, 16), (128, 48, 8, 256), (128, 10, 10, 64),
          (64, 12, 4, 32)]


@pytest.mark.parametrize("D,Hq,Hkv,bs", SHAPES)
def test_single_split_equals_two_step_and_oracle(D, Hq, Hkv, bs):
    rng = np.random.default_rng(1000 + D + Hq + bs)
    lens = [0, 1, 17, 200, 513, 64, 5]
    q, kp, vp, tables, n = _case(rng, lens, Hq, Hkv, D, bs)
    max_len = int(n.max())
    split = (max_len + 63) // 64 * 64
    assert pkv.decode_split_tokens(len(lens), Hq, Hkv, max_len, split) == split
    say(f"single split D={D} Hq={Hq} Hkv={Hkv} bs={bs} split={split}")
    qd, kc, vc, td, nd = dev_u16(q), dev_u16(kp), dev_u16(vp), dev_i32(tables), dev_i32(n)
    direct = pkv.paged_decode_attention(qd, kc, vc, td, nd, max_len, split_tokens=split)
    ws = torch.empty(pkv.decode_workspace_bytes(len(lens), Hq, Hkv, D, max_len, split),
                     dtype=torch.uint8, device="cuda")
    pkv.decode_attention_partial(qd, kc, vc, td, nd, max_len, ws, split_tokens=split)
    two = torch.empty_like(direct)
    pkv.decode_attention_reduce(two, nd, Hkv, tables.shape[1], bs, max_len, ws, split_tokens=split)
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(direct), host_u16(two))
    got = bf16_out_to_f64(direct)
    assert not got[0].any(), "an empty row's output is the zero vector"
    ref = oracle.decode_attention(q, kp, vp, tables, n)
    err = float(np.abs(got - ref).max())
    say(f"  max abs err {err:.3e}")
    assert err <= ATTN_TOL


@pytest.mark.parametrize("D,Hq,Hkv,bs", [SHAPES[0], SHAPES[2], SHAPES[4]])
def test_single_split_fused_store(D, Hq, Hkv, bs):
    """Fused store + single split: pools as after a separate store, output
    equal to the unfused single-split attention over the stored pools."""
    rng = np.random.default_rng(2000 + D + Hq + bs)
    lens = [3, 0, 130, 511, 64]
    q, kp, vp, tables, n = _case(rng, lens, Hq, Hkv, D, bs)
    kn, vn = _normal_bf16(rng, (len(lens), Hkv, D)), _normal_bf16(rng, (len(lens), Hkv, D))
    max_len = int(n.max())
    split = (max_len + 63) // 64 * 64
    say(f"single split fused D={D} Hq={Hq} Hkv={Hkv} bs={bs}")
    qd, td, nd = dev_u16(q), dev_i32(tables), dev_i32(n)
    kc, vc = dev_u16(kp), dev_u16(vp)
    fused = pkv.paged_decode_attention_store(qd, kc, vc, dev_u16(kn), dev_u16(vn), td, nd, max_len,
                                             split_tokens=split)
    slots = oracle.slot_mapping(tables, n, bs)
    kref, vref = kp.copy(), vp.copy()
    assert oracle.kv_store(kref, vref, kn, vn, slots, bs) == 0
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(kc), kref) and np.array_equal(host_u16(vc), vref)
    plain = pkv.paged_decode_attention(qd, dev_u16(kref), dev_u16(vref), td, nd, max_len,
                                       split_tokens=split)
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(fused), host_u16(plain))
    ref = oracle.decode_attention(q, kref, vref, tables, n)
    assert float(np.abs(bf16_out_to_f64(fused) - ref).max()) <= ATTN_TOL
