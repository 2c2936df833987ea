"""A decode step captured as a HIP graph must give the eager results on every
replay.  Replays are interleaved with eager work and synchronisations, and
each replay's outputs are compared bit for bit with the eager step (all
kernels are deterministic)."""
import numpy as np
import pytest
import torch

import paged_kv_decode_store_amd as pkv
from workloads import config_by_name, host_inputs

from gpu_util import dev_f32, dev_i32, dev_u16, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_decode_step_graph_replays_match_eager():
    cfg = config_by_name("tiny")
    inp = host_inputs(cfg, layers=(0,))
    n, t = inp.context_lens, inp.block_tables
    kc, vc = dev_u16(inp.k_pool[0]), dev_u16(inp.v_pool[0])
    nd, td = dev_i32(n), dev_i32(t)
    q, kn, vn = dev_u16(inp.q[0]), dev_u16(inp.k_new[0]), dev_u16(inp.v_new[0])
    z, g = dev_f32(inp.logits), dev_f32(inp.gumbel)
    B = cfg.batch
    # exercise every sampler pass: mixed greedy / top-k / top-p rows
    temp = dev_f32(np.array([0.7, 0.0, 1.0, 0.9], np.float32))
    top_p = dev_f32(np.array([0.9, 1.0, 0.8, 1.0], np.float32))
    top_k = dev_i32(np.array([0, 0, 40, 7], np.int32))
    max_len = int(n.max())
    ws = torch.empty(pkv.decode_workspace_bytes(B, cfg.num_q_heads, cfg.num_kv_heads,
                                                cfg.head_dim, max_len), dtype=torch.uint8,
                     device="cuda")
    sws = torch.empty(pkv.sampler_workspace_bytes(B, cfg.vocab), dtype=torch.uint8, device="cuda")
    slots = torch.empty(B, dtype=torch.int32, device="cuda")
    out = torch.empty((B, cfg.num_q_heads, cfg.head_dim), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty(B, dtype=torch.int32, device="cuda")

    def step():
        pkv.slot_mapping(td, nd, cfg.block_size, out=slots)
        pkv.kv_store(kc, vc, kn, vn, slots)
        pkv.paged_decode_attention(q, kc, vc, td, nd, max_len, out=out, workspace=ws)
        pkv.sample_next_token(z, g, temp, top_p, top_k, out=ids, workspace=sws)

    say("graph: eager reference")
    step()
    torch.cuda.synchronize()
    ref_out, ref_ids, ref_slots = out.clone(), ids.clone(), slots.clone()
    ref_k = kc.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for r in range(4):
        # unrelated eager work on the same buffers between replays
        out.zero_()
        ids.fill_(-7)
        slots.fill_(-3)
        ws.fill_(0xAB)
        sws.fill_(0xCD)
        torch.cuda.synchronize()
        say(f"graph: replay {r}")
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), r
        assert torch.equal(ids, ref_ids), r
        assert torch.equal(slots, ref_slots), r
        assert torch.equal(kc.view(torch.int16), ref_k.view(torch.int16)), r
        # an eager step in between must still agree too
        step()
        torch.cuda.synchronize()
        assert torch.equal(ids, ref_ids) and torch.equal(out.view(torch.int16),
                                                         ref_out.view(torch.int16))
