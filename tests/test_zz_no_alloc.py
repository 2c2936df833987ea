"""GPU: the no-allocation attention entry point against the one it varies.

pkv_paged_decode_attention_store_noalloc keeps its split-KV partials in the
library's fixed device array instead of a caller workspace.  Through the C
ABI it must reproduce pkv_paged_decode_attention_store bit for bit (same
kernels, same arguments), outputs and stored pools alike, and stay within
the attention bar of the fp64 oracle: on two calls in a row, the second
smaller than the first (the array keeps the first call's contents), on the
VALU and the matrix-core kernels, with several splits per row.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_store_amd as pkv
from workloads.generate import bf16_bits_from_f32

from gpu_util import ATTN_TOL, dev_i32, dev_u16, host_u16, oracle_heads, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _bf16(rng, shape):
    return bf16_bits_from_f32(rng.standard_normal(size=shape, dtype=np.float32))


def _case(seed, B, Hq, Hkv, D, bs, lo, hi):
    rng = np.random.default_rng(seed)
    n = rng.integers(lo, hi + 1, size=B).astype(np.int32)
    n[0] = hi
    need = (n.astype(np.int64) + bs - 1) // bs
    nb = int(need.sum()) + 3
    perm = rng.permutation(nb).astype(np.int32)
    t = np.zeros((B, int(need.max())), np.int32)
    pos = 0
    for b in range(B):
        t[b, :need[b]] = perm[pos:pos + need[b]]
        pos += need[b]
    return (n, t, _bf16(rng, (nb, bs, Hkv, D)), _bf16(rng, (nb, bs, Hkv, D)),
            _bf16(rng, (B, Hq, D)), _bf16(rng, (B, Hkv, D)), _bf16(rng, (B, Hkv, D)))


def _both(case, split):
    n, t, kp, vp, q, kn, vn = case
    B, Hq, D = q.shape
    max_len = int(n.max())
    res = []
    for which in ("workspace", "noalloc"):
        kc, vc = dev_u16(kp), dev_u16(vp)
        out = torch.full((B, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        args = (dev_u16(q), kc, vc, dev_u16(kn), dev_u16(vn), dev_i32(t), dev_i32(n), max_len)
        if which == "workspace":
            pkv.paged_decode_attention_store(*args, split_tokens=split, out=out)
        else:
            pkv.paged_decode_attention_store_noalloc(*args, out=out, split_tokens=split)
        torch.cuda.synchronize()
        res.append((host_u16(out), host_u16(kc), host_u16(vc)))
    return res


@pytest.mark.parametrize("Hq,Hkv", [(16, 8), (48, 8)], ids=["valu", "mfma"])
def test_noalloc_equals_workspace_entry_point_twice(Hq, Hkv):
    big = _case(11, 48, Hq, Hkv, 128, 256, 500, 4096)
    small = _case(12, 5, Hq, Hkv, 128, 16, 1, 700)
    for label, case, split in (("large", big, 0), ("small", small, 64)):
        n, t, kp, vp, q, kn, vn = case
        B = len(n)
        s = pkv.decode_split_tokens(B, Hq, Hkv, int(n.max()), split)
        need = pkv.decode_workspace_bytes(B, Hq, Hkv, 128, int(n.max()), split)
        say(f"noalloc {label}: B={B} Hq={Hq} split {s}, partials {need} bytes")
        assert need <= pkv._lib.PKV_STATIC_SCRATCH_BYTES
        assert -(-int(n.max()) // s) > 1        # several splits: the array is used
        (o_ws, k_ws, v_ws), (o_na, k_na, v_na) = _both(case, split)
        assert np.array_equal(o_na, o_ws), label
        assert np.array_equal(k_na, k_ws) and np.array_equal(v_na, v_ws), label
        kref, vref = kp.copy(), vp.copy()
        assert oracle.kv_store(kref, vref, kn, vn, oracle.slot_mapping(t, n, kp.shape[1]),
                               kp.shape[1]) == 0
        assert np.array_equal(k_na, kref) and np.array_equal(v_na, vref)
        g = Hq // Hkv
        ref = oracle_heads(q, kref, vref, t, n, [(b, h) for b in range(B) for h in range(Hq)], g)
        got = (o_na.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        err = max(float(np.abs(got[b, h] - r).max()) for (b, h), r in ref.items())
        say(f"  max abs err vs oracle {err:.3e}")
        assert err <= ATTN_TOL


def test_noalloc_rejects_partials_beyond_the_array():
    """64 rows x 64 heads at 131072 positions need ~90 MB of partials: the
    call is refused on the host, before any launch (so the stand-in pool,
    queries and lengths here are never read)."""
    B, Hq, Hkv, D, bs, L = 64, 64, 8, 128, 256, 131072
    assert pkv.decode_workspace_bytes(B, Hq, Hkv, D, L) > pkv._lib.PKV_STATIC_SCRATCH_BYTES
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((4, bs, Hkv, D), dtype=torch.bfloat16, device="cuda")
    kn = torch.zeros((B, Hkv, D), dtype=torch.bfloat16, device="cuda")
    t = torch.zeros((B, L // bs), dtype=torch.int32, device="cuda")
    n = torch.full((B,), L, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(pkv.PkvError) as e:
        pkv.paged_decode_attention_store_noalloc(q, kc, kc.clone(), kn, kn.clone(), t, n, L,
                                                 out=out)
    assert e.value.status == pkv._lib.PKV_ERR_WORKSPACE
