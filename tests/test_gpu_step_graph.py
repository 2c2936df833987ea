"""GPU: the benchmarked decode step, captured as one HIP graph and replayed,
against the oracle.

The step is the benchmark's own call sequence (paged_kv_decode_store_amd.
step.decode_step, the nano-vllm "run model" order): for every layer the
fused store + attention partial step and the reduce, then the sampler.  It
is captured once and replayed three times with unrelated eager work in
between; every replay must reproduce the first bit for bit, the stored
pools must equal the oracle's store bit for bit, the checked layers'
outputs must be within the attention bar of the fp64 oracle, and the ids
must equal the oracle's exactly.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_store_amd as pkv
from paged_kv_decode_store_amd.step import SamplerArgs, decode_step
from workloads import config_by_name, host_inputs
from workloads.device import device_pool
from workloads.generate import sampling_params

from gpu_util import (ATTN_TOL, compare_ids, dev_f32, dev_i32, dev_u16, host_u16, oracle_heads,
                      say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


@pytest.mark.parametrize("name,check_layers", [("qwen3", (0, 9, 18, 27)), ("long", (0,))],
                         ids=["qwen3", "long"])
def test_benchmarked_step_graph_matches_oracle(name, check_layers):
    cfg = config_by_name(name)
    L = cfg.num_layers
    B, Hq, Hkv, D, bs = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    inp = host_inputs(cfg, layers=range(L), pools=False, sampler=True)
    n, t = inp.context_lens, inp.block_tables
    nd, td = dev_i32(n), dev_i32(t)
    max_len = int(n.max())
    say(f"step graph {name}: {L} layers, B={B}")
    kp = [device_pool(cfg, inp.num_blocks, "kpool", l) for l in range(L)]
    vp = [device_pool(cfg, inp.num_blocks, "vpool", l) for l in range(L)]
    # host copies of the checked layers' pools before the step
    k0 = {l: host_u16(kp[l]) for l in check_layers}
    v0 = {l: host_u16(vp[l]) for l in check_layers}
    layers = [(dev_u16(inp.q[l]), kp[l], vp[l], dev_u16(inp.k_new[l]), dev_u16(inp.v_new[l]))
              for l in range(L)]
    outs = [torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    split = pkv.decode_split_tokens(B, Hq, Hkv, max_len)
    ws = torch.empty(pkv.decode_workspace_bytes(B, Hq, Hkv, D, max_len, split), dtype=torch.uint8,
                     device="cuda")
    tt, pp, kk = sampling_params(cfg)
    samp = SamplerArgs(dev_f32(inp.logits), dev_f32(inp.gumbel), dev_f32(tt), dev_f32(pp),
                       dev_i32(kk), torch.empty(B, dtype=torch.int32, device="cuda"),
                       torch.empty(pkv.sampler_workspace_bytes(B, cfg.vocab), dtype=torch.uint8,
                                   device="cuda"))

    def run():
        decode_step(layers, td, nd, bs, max_len, out=outs, workspace=ws, split_tokens=split,
                    sampler=samp)

    # as the benchmark: one call on a side stream, then the capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()

    first = None
    for r in range(3):
        for o in outs:
            o.fill_(0)
        samp.ids.fill_(-5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = ([host_u16(outs[l]) for l in check_layers], samp.ids.cpu().numpy().copy())
        say(f"  replay {r} done")
        if first is None:
            first = got
        else:
            for a, b in zip(first[0], got[0]):
                assert np.array_equal(a, b), f"replay {r} differs from replay 0"
            assert np.array_equal(first[1], got[1])
        # unrelated eager work between replays
        x = torch.randn(1 << 20, device="cuda")
        (x * 2).sum().item()

    for i, l in enumerate(check_layers):
        kref, vref = k0[l], v0[l]
        slots = oracle.slot_mapping(t, n, bs)
        assert oracle.kv_store(kref, vref, inp.k_new[l], inp.v_new[l], slots, bs) == 0
        assert np.array_equal(host_u16(kp[l]), kref), f"layer {l}: K pool"
        assert np.array_equal(host_u16(vp[l]), vref), f"layer {l}: V pool"
        got = _bf16_to_f64(first[0][i])
        if name == "long":
            # one query head per KV head of every row, at varying places in
            # the group (the full 512 heads would take the oracle minutes)
            pairs = [(b, kvh * cfg.group + (b + kvh) % cfg.group) for b in range(B)
                     for kvh in range(Hkv)]
        else:
            pairs = [(b, h) for b in range(B) for h in range(Hq)]   # every output
        ref = oracle_heads(inp.q[l], kref, vref, t, n, pairs, cfg.group)
        err = max(float(np.abs(got[b, h] - ref[(b, h)]).max()) for b, h in pairs)
        say(f"  layer {l}: max abs err {err:.3e} over {len(pairs)} (row, head) pairs")
        assert err <= ATTN_TOL
    ref_ids, infos = oracle.sample(inp.logits, inp.gumbel, tt, pp, kk)
    bad, amb = compare_ids(first[1], ref_ids, infos)
    assert not bad and amb == 0, (bad, amb)


def _bf16_to_f64(u16):
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
