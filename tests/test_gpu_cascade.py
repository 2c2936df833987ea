"""GPU parity of the shared-prefix (cascade) decode against the CPU oracle.

The cascade reads the blocks that every row shares once per KV head and
merges them with each row's own positions; its result is defined as the
plain paged decode attention over each whole row, so the oracle is the
ordinary fp64 decode attention over the full block tables.  Bar: max-abs
1e-2, zero output for empty rows.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_store_amd as pkv
from workloads import config_by_name, host_inputs
from workloads.generate import bf16_bits_from_f32

from gpu_util import ATTN_TOL, bf16_out_to_f64, dev_i32, dev_u16, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _normal_bf16(rng, shape):
    return bf16_bits_from_f32(rng.standard_normal(size=shape, dtype=np.float32))


def _shared_prefix_case(rng, Hq, Hkv, D, bs, npb, lens, spare=2):
    """Rows whose first npb logical blocks are the same physical blocks,
    then private blocks from a permutation of the rest of the pool."""
    lens = np.asarray(lens, np.int32)
    B = len(lens)
    need = [max(npb, (int(n) + bs - 1) // bs) for n in lens]
    W = max(need)
    private = [x - npb for x in need]
    nb = npb + sum(private) + spare
    perm = rng.permutation(nb).astype(np.int32)
    shared = perm[:npb]
    tables = np.full((B, W), -1, np.int32)
    pos = npb
    for b in range(B):
        tables[b, :npb] = shared
        tables[b, npb:need[b]] = perm[pos:pos + private[b]]
        pos += private[b]
    kp, vp = _normal_bf16(rng, (nb, bs, Hkv, D)), _normal_bf16(rng, (nb, bs, Hkv, D))
    q = _normal_bf16(rng, (B, Hq, D))
    return q, kp, vp, shared, tables, lens


def _run_cascade(q, kp, vp, shared, tables, lens, split=0):
    maxlen = int(max(1, lens.max()))
    out = pkv.cascade_decode_attention(dev_u16(q), dev_u16(kp), dev_u16(vp), dev_i32(shared),
                                       dev_i32(tables), dev_i32(lens), maxlen,
                                       split_tokens=split)
    torch.cuda.synchronize()
    return bf16_out_to_f64(out)


@pytest.mark.parametrize("D,Hq,Hkv,bs,npb,lens,split", [
    # rows shorter than, equal to and longer than the prefix, and an empty row
    (128, 4, 2, 16, 3, [0, 10, 48, 49, 200], 0),
    (64, 6, 2, 32, 2, [64, 65, 1, 300, 64, 129, 5], 64),   # 21 virtual queries per KV head
    (128, 10, 10, 256, 4, [1025, 1100, 1281, 1030], 0),
    (128, 16, 1, 16, 5, [80, 81, 95, 400, 17, 79], 128),   # group 16: 96 virtual queries
    (64, 8, 8, 64, 1, [64, 65, 66, 640, 2000], 192),
    (128, 8, 2, 16, 8, [128] * 3 + [129] * 3, 0),          # tails of exactly one position
])
def test_cascade_matches_oracle(D, Hq, Hkv, bs, npb, lens, split):
    rng = np.random.default_rng(D + 3 * Hq + 5 * Hkv + bs + npb + len(lens))
    q, kp, vp, shared, tables, lens = _shared_prefix_case(rng, Hq, Hkv, D, bs, npb, lens)
    say(f"cascade D={D} Hq={Hq} Hkv={Hkv} bs={bs} prefix_blocks={npb} split={split} "
        f"lens={lens.tolist()}")
    got = _run_cascade(q, kp, vp, shared, tables, lens, split)
    ref = oracle.decode_attention(q, kp, vp, tables, lens)
    err = np.abs(got - ref).max()
    say(f"  max abs err {err:.3e}")
    assert err <= ATTN_TOL
    for b in np.nonzero(lens == 0)[0]:
        assert np.all(got[b] == 0.0)


def test_cascade_clone_workload_decode_step():
    """The 16-way clone workload: slot mapping + store on the GPU, then the
    cascade attention, against the oracle's store + attention."""
    cfg = config_by_name("clone")
    inp = host_inputs(cfg, layers=(0,), sampler=False)
    n, t = inp.context_lens, inp.block_tables
    pre = cfg.clone_prefix_blocks
    assert np.all(t[:, :pre] == t[0, :pre])
    kc, vc = dev_u16(inp.k_pool[0]), dev_u16(inp.v_pool[0])
    nd, td = dev_i32(n), dev_i32(t)
    say("cascade clone decode step")
    slots = pkv.slot_mapping(td, nd, cfg.block_size)
    pkv.kv_store(kc, vc, dev_u16(inp.k_new[0]), dev_u16(inp.v_new[0]), slots)
    out = pkv.cascade_decode_attention(dev_u16(inp.q[0]), kc, vc, dev_i32(t[0, :pre]), td, nd,
                                       int(n.max()))
    plain = pkv.paged_decode_attention(dev_u16(inp.q[0]), kc, vc, td, nd, int(n.max()))
    torch.cuda.synchronize()
    kref, vref = inp.k_pool[0].copy(), inp.v_pool[0].copy()
    oracle.kv_store(kref, vref, inp.k_new[0], inp.v_new[0],
                    oracle.slot_mapping(t, n, cfg.block_size), cfg.block_size)
    ref = oracle.decode_attention(inp.q[0], kref, vref, t, n)
    got = bf16_out_to_f64(out)
    err = np.abs(got - ref).max()
    say(f"  max abs err {err:.3e}")
    assert err <= ATTN_TOL
    assert np.abs(got - bf16_out_to_f64(plain)).max() <= ATTN_TOL


def test_cascade_workspace_reuse_and_graph_replay():
    """A workspace reused across calls with different lengths, and the
    cascade captured in a HIP graph, replayed with eager work in between."""
    rng = np.random.default_rng(5)
    q, kp, vp, shared, tables, lens = _shared_prefix_case(rng, 8, 4, 128, 16, 4,
                                                          [70, 64, 300, 65, 0, 129])
    qd, kd, vd = dev_u16(q), dev_u16(kp), dev_u16(vp)
    sd, td, nd = dev_i32(shared), dev_i32(tables), dev_i32(lens)
    maxlen = int(lens.max())
    ws = torch.empty(pkv.cascade_workspace_bytes(6, 8, 4, 128, maxlen, 4, 16), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((6, 8, 128), dtype=torch.bfloat16, device="cuda")
    ref = oracle.decode_attention(q, kp, vp, tables, lens)
    # a shorter call first leaves different partials in the workspace
    short = np.minimum(lens, 64).astype(np.int32)
    pkv.cascade_decode_attention(qd, kd, vd, sd, td, dev_i32(short), maxlen, out=out, workspace=ws)
    pkv.cascade_decode_attention(qd, kd, vd, sd, td, nd, maxlen, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert np.abs(bf16_out_to_f64(out) - ref).max() <= ATTN_TOL
    eager = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pkv.cascade_decode_attention(qd, kd, vd, sd, td, nd, maxlen, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        pkv.cascade_decode_attention(qd, kd, vd, sd, td, nd, maxlen, out=out, workspace=ws)
    for r in range(3):
        out.zero_()
        ws.fill_(0x7F)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), r
