"""Decode-step benchmark on one MI355X.

One step = slot mapping, then for each of L layers the KV store and the
split-KV paged decode attention (partial + reduce), then the sampler over
the logits.  Default workload: the Qwen3-0.6B-shaped decode (64 rows,
contexts uniform in [128, 4096], GQA 16/8, head_dim 128, block 256,
28 layers, vocab 151936, T 0.8, top-p 0.95), synthetic seeded inputs
resident in HBM before timing starts.

Prints ONE JSON line.  `value` is the paged decode-attention throughput in
GB/s of algorithmic bytes (each distinct cached K/V element once + Q + O,
per layer) over the attention time per layer, measured by replaying the
L layers' partial + reduce launches as a HIP graph between two HIP events.
Decode steps/s (whole step replayed as a graph) and sampler tokens/s ride
along, with per-kernel HIP-event times of eager steps.  `roofline` covers
the dominant kernel (the attention partial step): its average launch time
from a graph of the L partial launches alone.  `cpu_baseline` times the
CPU oracle on a bounded sample of the same workload.  Workloads small
enough to sit in the 256 MB Infinity Cache cycle over copies of their
pools so that each step reads from HBM; their warm (same pools) figure is
reported beside it.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
WORKLOAD_TITLES = {
    "tiny": "tiny: 4 rows, contexts 17/256/299/513, MHA 16 heads x 64, vocab 32768",
    "qwen3": "qwen3: Qwen3-0.6B-shaped paged decode step",
    "grok": "grok: Grok-1-shaped attention, 32 rows x 2048 positions, GQA 48/8, contiguous tables",
    "clone": "clone: 16-way clone, 4 shared prefix blocks + private tails, MHA 10 heads, top-k 50",
    "long": "long: 8 rows, contexts 32k-128k, GQA 64/8, fragmented pool",
}
ROOT = os.path.dirname(os.path.abspath(__file__))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="qwen3")
    ap.add_argument("--split", type=int, default=0, help="split_tokens (0 = automatic)")
    ap.add_argument("--layers", type=int, default=0, help="override layer count (0 = workload's)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline (0 disables it)")
    ap.add_argument("--unfused", action="store_true",
                    help="separate slot-mapping and store launches instead of the fused "
                         "store + attention partial")
    ap.add_argument("--cascade", action="store_true",
                    help="shared-prefix workloads: the cascade decode (prefix read once for "
                         "all rows) instead of the plain paged attention")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches only (no HIP-graph replay of the step)")
    ap.add_argument("--calibrate-copy", type=int, default=0,
                    help="also run a device copy of this many MiB (counter calibration)")
    ap.add_argument("--rotate", type=int, default=0,
                    help="independent copies of the pools, cycled step by step so that at "
                         "least 1 GB of cache is touched between reuses (0 = automatic)")
    ap.add_argument("--varlen", default="",
                    help="time varlen multi-query (chunked prefill) attention on this "
                         "workload instead of the decode step (qwen3_prefill)")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="host threads for the oracle baseline (0 = the CPUs this process "
                         "may use, at most 16)")
    return ap.parse_args()


def unique_positions(n, tables, bs):
    """Distinct physical slots read by all rows (shared prefix blocks once)."""
    seen = set()
    for b in range(len(n)):
        nb = int(n[b])
        for j in range((nb + bs - 1) // bs):
            used = min(bs, nb - j * bs)
            seen.update(int(tables[b][j]) * bs + o for o in range(used))
    return len(seen)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    sys.path.insert(0, ROOT)
    import paged_kv_decode_store_amd as pkv
    from paged_kv_decode_store_amd.step import CascadeArgs, SamplerArgs, decode_step
    from workloads import config_by_name, host_inputs
    from workloads.device import device_pool
    from workloads.generate import sampling_params

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    pkv.lib()  # fail loudly if the HIP library is missing
    if args.varlen:
        run_varlen(args)
        return

    cfg = config_by_name(args.config)
    L = args.layers or cfg.num_layers
    B, Hq, Hkv, D, bs = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    log(f"[bench] workload {cfg.name}: B={B} Hq={Hq} Hkv={Hkv} D={D} bs={bs} L={L} V={cfg.vocab}")

    inp = host_inputs(cfg, layers=range(L), pools=False, sampler=True)
    n, tables = inp.context_lens, inp.block_tables
    dev = torch.device("cuda")

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    nd, td = i32(n), i32(tables)
    q = [bf16(x) for x in inp.q]
    kn = [bf16(x) for x in inp.k_new]
    vn = [bf16(x) for x in inp.v_new]
    # cache hygiene: workloads whose pools fit in the 256 MB Infinity Cache
    # cycle over R copies so that >= 1 GB is touched between two reuses
    uniq = unique_positions(n, tables, bs)
    touched = uniq * Hkv * D * 4 * L
    R = args.rotate or max(1, min(256, -(-1_000_000_000 // touched)))
    kp, vp = [], []   # [copy][layer]
    for c in range(R):
        if c == 0:
            kp.append([device_pool(cfg, inp.num_blocks, "kpool", layer) for layer in range(L)])
            vp.append([device_pool(cfg, inp.num_blocks, "vpool", layer) for layer in range(L)])
        else:
            kp.append([x.clone() for x in kp[0]])
            vp.append([x.clone() for x in vp[0]])
    logits = torch.from_numpy(inp.logits).to(dev)
    gumbel = torch.from_numpy(inp.gumbel).to(dev)
    t, p, k = (torch.from_numpy(x).to(dev) for x in sampling_params(cfg))
    max_len = int(n.max())
    split = pkv.decode_split_tokens(B, Hq, Hkv, max_len, args.split)
    ws = torch.empty(pkv.decode_workspace_bytes(B, Hq, Hkv, D, max_len, split), dtype=torch.uint8,
                     device=dev)
    sws = torch.empty(pkv.sampler_workspace_bytes(B, cfg.vocab), dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    slots = torch.empty(B, dtype=torch.int32, device=dev)
    ids = torch.empty(B, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs resident: {sum(x.numel() * 2 for c in range(R) for x in kp[c] + vp[c]) / 1e9:.2f} GB "
        f"of pools ({R} cop{'y' if R == 1 else 'ies'}), split_tokens={split}")

    # rows sharing their first blocks (the clone workload): cascade decode,
    # the shared prefix read once per KV head for all rows
    cascade = cfg.clone_prefix_blocks > 0 and args.cascade
    fused = not args.unfused and not cascade
    if cascade:
        prefix = i32(tables[0, :cfg.clone_prefix_blocks])
        cws = torch.empty(pkv.cascade_workspace_bytes(B, Hq, Hkv, D, max_len,
                                                      cfg.clone_prefix_blocks, bs, args.split),
                          dtype=torch.uint8, device=dev)

    def partial(layer, c):
        K, V = kp[c][layer], vp[c][layer]
        if cascade:
            pkv.cascade_decode_attention(q[layer], K, V, prefix, td, nd, max_len, out=out,
                                         workspace=cws, split_tokens=args.split)
        elif fused:
            # store of the new K/V fused into the attention partial step
            pkv.decode_attention_partial_store(q[layer], K, V, kn[layer], vn[layer], td, nd,
                                               max_len, ws, split_tokens=split)
        else:
            pkv.decode_attention_partial(q[layer], K, V, td, nd, max_len, ws,
                                         split_tokens=split)

    def reduce():
        if not cascade:  # the cascade call includes its reduce
            pkv.decode_attention_reduce(out, nd, Hkv, tables.shape[1], bs, max_len, ws,
                                        split_tokens=split)

    # the step itself: one fixed sequence of library calls shared with the
    # step tests (paged_kv_decode_store_amd.step.decode_step)
    layer_args = [[(q[l], kp[c][l], vp[c][l], kn[l], vn[l]) for l in range(L)] for c in range(R)]
    samp = SamplerArgs(logits, gumbel, t, p, k, ids, sws)
    mode = "cascade" if cascade else "fused" if fused else "unfused"
    casc = CascadeArgs(prefix, cws) if cascade else None

    def step(ev=None, c=0):
        mark = None
        if ev is not None:
            def mark(point, layer):
                {"partial": lambda: ev["p0"][layer], "reduce": lambda: ev["p1"][layer],
                 "done": lambda: ev["r1"][layer], "sampler": lambda: ev["s0"],
                 "end": lambda: ev["s1"]}[point]().record()
        decode_step(layer_args[c], td, nd, bs, max_len, out=out, workspace=ws,
                    split_tokens=args.split if cascade else split, sampler=samp, mode=mode,
                    slots=slots, cascade=casc, mark=mark)

    for i in range(args.warmup):
        step(c=i % R)
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps)")

    def new_events():
        E = lambda: torch.cuda.Event(enable_timing=True)
        return {"p0": [E() for _ in range(L)], "p1": [E() for _ in range(L)],
                "r1": [E() for _ in range(L)], "s0": E(), "s1": E()}

    # timed region: K whole steps, per-kernel events recorded on the same stream
    evs = [new_events() for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(evs[i], c=i % R)
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    part_ms = [e["p0"][l].elapsed_time(e["p1"][l]) for e in evs for l in range(L)]
    red_ms = [e["p1"][l].elapsed_time(e["r1"][l]) for e in evs for l in range(L)]
    samp_ms = [e["s0"].elapsed_time(e["s1"]) for e in evs]
    log(f"[bench] timed {args.steps} eager steps in {total_ms:.2f} ms")
    eager_ms_per_step = total_ms / args.steps


    # the same step captured once as a HIP graph and replayed: removes the
    # host launch gaps between the ~3L+10 kernels of a step
    def attention_only(c, with_reduce=True):
        for layer in range(L):
            partial(layer, c)
            if with_reduce:
                reduce()

    def graph_time_ms(fn, ncalls=None):
        """Capture R consecutive calls fn(c), c = 0..R-1 (one per pool copy;
        `ncalls` of them if given), as one HIP graph; return the replayed time
        per call in ms."""
        nc = R if ncalls is None else ncalls
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn(0)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for c in range(nc):
                fn(c)
        for _ in range(max(1, args.warmup // nc)):
            graph.replay()
        torch.cuda.synchronize()
        reps = max(1, args.steps // nc)
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(reps):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        return g0.elapsed_time(g1) / (reps * nc)

    # HIP-graph replay, as a serving engine runs a decode step: removes the
    # host launch gaps between kernels.  Three graphs: the whole step, the
    # attention alone (L x (partial + reduce)) and the partial kernels alone.
    graph_ms_per_step = graph_attn_us = graph_part_us = None
    if not args.no_graph:
        graph_ms_per_step = graph_time_ms(lambda c: step(c=c))
        graph_attn_us = 1e3 * graph_time_ms(lambda c: attention_only(c)) / L
        graph_part_us = 1e3 * graph_time_ms(lambda c: attention_only(c, with_reduce=False)) / L
        log(f"[bench] graph replays: {graph_ms_per_step:.4f} ms per step, attention "
            f"{graph_attn_us:.2f} us per layer, partial {graph_part_us:.2f} us per launch")
    # The sampler alone as a graph replay (as the step graph runs it), over
    # enough copies of the logits (up to 64) that each draw reads its logits
    # from HBM as it would after a step's attention.
    graph_samp_us = None
    samp_copies = 1
    if not args.no_graph:
        samp_copies = int(min(64, max(1, -(-(1 << 30) // (logits.numel() * 4)))))
        lcopies = [logits] + [logits.clone() for _ in range(samp_copies - 1)]
        graph_samp_us = 1e3 * graph_time_ms(
            lambda c: pkv.sample_next_token(lcopies[c], gumbel, t, p, k, out=ids,
                                            workspace=sws), ncalls=samp_copies)
        del lcopies
        log(f"[bench] sampler graph replay: {graph_samp_us:.2f} us per draw "
            f"({samp_copies} logits copies)")
    # The reduce's floor: one launch that only streams the workspace holding
    # the split partials (all splits; the reduce reads a row's used ones),
    # timed as a graph of at least 64 such launches (fewer would time the
    # host's replay calls, not the device).
    reduce_floor = None
    if not args.no_graph and not cascade:
        pbytes = (ws.numel() // 16) * 16
        sink = torch.zeros(64, dtype=torch.int32, device=dev)
        fl_us = 1e3 * graph_time_ms(
            lambda c: pkv.probe_stream_read(ws[:pbytes], sink), ncalls=max(L, 64))
        reduce_floor = {"us": round(fl_us, 3), "bytes": pbytes,
                        "what": "pkv_probe_stream_read over the partials workspace (16 "
                                "workgroups per CU), graph replay: a launch that only reads "
                                "what the reduce reads"}
        log(f"[bench] reduce floor: {fl_us:.2f} us per launch")
    warm_attn_us = None
    if R > 1 and not args.no_graph:
        # the same pools every time: what a cache-resident workload reaches
        warm_attn_us = 1e3 * graph_time_ms(lambda c: attention_only(0)) / L

    # algorithmic bytes: K and V of every distinct cached position once (a
    # shared prefix counts once), + Q + O
    kv_logical = int(n.astype(np.int64).sum()) * Hkv * D * 2 * 2
    kv_bytes = uniq * Hkv * D * 2 * 2
    q_bytes = B * Hq * D * 2
    o_bytes = B * Hq * D * 2
    attn_bytes_layer = kv_bytes + q_bytes + o_bytes
    part_ev_us = 1e3 * float(np.mean(part_ms))
    red_ev_us = 1e3 * float(np.mean(red_ms))
    attn_us_layer = graph_attn_us if graph_attn_us is not None else part_ev_us + red_ev_us
    part_avg_us = graph_part_us if graph_part_us is not None else part_ev_us
    value = attn_bytes_layer / (attn_us_layer * 1e-6) / 1e9
    store_bytes = 2 * B * Hkv * D * 2 if fused else 0   # new K and V rows written
    part_bytes = kv_bytes + q_bytes + store_bytes
    part_gbs = part_bytes / (part_avg_us * 1e-6) / 1e9
    ms_per_step = graph_ms_per_step if graph_ms_per_step is not None else eager_ms_per_step
    samp_eager_us = 1e3 * float(np.mean(samp_ms))
    samp_avg_us = graph_samp_us if graph_samp_us is not None else samp_eager_us
    traffic = read_traffic(cfg.name, fused, cfg.group >= 3)

    # The device as the runtime reports it, and the streaming-read rate it
    # sustains with the attention kernels' loads: the ceiling the partial
    # kernel's rate is held against beside the nominal 8 TB/s.
    device = pkv.device_info(torch.cuda.current_device())
    ceiling = stream_read_ceiling(dev)
    log(f"[bench] streaming-read ceiling {ceiling['GBps']:.0f} GB/s")

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(cfg, inp, kp[0][0], vp[0][0], args.cpu_seconds, args.cpu_threads)

    if args.calibrate_copy > 0:
        nbytes = args.calibrate_copy << 20
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {nbytes} bytes done")

    res = {
        "metric": "paged decode-attn HBM GB/s (% of peak) + decode steps/s; sampler tokens/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TITLES.get(cfg.name, cfg.name),
                   "batch": B, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D,
                   "block_size": bs, "layers": L, "vocab": cfg.vocab,
                   "context_tokens": int(n.sum()), "split_tokens": split,
                   "temperature": cfg.temperature, "top_p": cfg.top_p, "top_k": cfg.top_k},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "decode_steps_per_s": round(1e3 / ms_per_step, 2),
        "step_timing": "hip_graph_replay" if graph_ms_per_step is not None else "eager",
        "ms_per_step_eager": round(eager_ms_per_step, 4),
        "sampler_tokens_per_s": round(B / (samp_avg_us * 1e-6), 1),
        "attention_us_per_layer": round(attn_us_layer, 3),
        "attention_timing": "hip_graph_replay" if graph_attn_us is not None else "hip_events",
        "eager_event_us_per_layer": {"partial": round(part_ev_us, 3), "reduce": round(red_ev_us, 3)},
        "reduce_us_per_layer": None if graph_attn_us is None or graph_part_us is None else
        round(graph_attn_us - graph_part_us, 3),
        "reduce_floor": reduce_floor,
        "sampler_us": round(samp_avg_us, 3),
        "sampler_timing": (f"hip_graph_replay over {samp_copies} logits copies"
                           if graph_samp_us is not None else "hip_events in the eager step"),
        "sampler_us_eager_step": round(samp_eager_us, 3),
        "kv_bytes_per_layer": {"unique": kv_bytes, "logical": kv_logical},
        "logical_GBps": round((kv_logical + q_bytes + o_bytes) / (attn_us_layer * 1e-6) / 1e9, 2),
        "cache": {"pool_copies_cycled": R,
                  "warm_attention_us_per_layer": None if warm_attn_us is None else
                  round(warm_attn_us, 3),
                  "warm_GBps": None if warm_attn_us is None else
                  round(attn_bytes_layer / (warm_attn_us * 1e-6) / 1e9, 2)},
        "step": ("slot mapping, store, cascade attention (shared prefix read once)" if cascade
                 else "fused store + attention" if fused else "slot mapping, store, attention"),
        "roofline": {"kernel": partial_kernel_name(cfg, D, fused, cascade),
                     "bound": "hbm", "achieved": round(part_gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(part_gbs / HBM_PEAK_GBS, 4),
                     "frac_of_stream_ceiling": round(part_gbs / ceiling["GBps"], 4),
                     "bytes_per_launch": part_bytes,
                     "avg_launch_us": round(part_avg_us, 3),
                     "launch_timing": "hip_graph_replay of the layers' partial launches"
                     if graph_part_us is not None else "hip_events per launch",
                     "traffic": traffic},
        "cpu_baseline": cpu,
        "device": device,
        "stream_read_ceiling": ceiling,
        # the pages' only tokens/s figure near this path: context, never the target
        "context": {"pages_anecdote": {
            "value": 32.0, "unit": "tokens/s",
            "what": "Grok-1 end-to-end decode on one A100 with light kernels and a static KV "
                    "cache, streaming ([xai] section 1); unverified, covers the whole model "
                    "including its weight reads, so not comparable to the attention-only value"}},
    }
    print(json.dumps(res), flush=True)


def run_varlen(args):
    """Chunked prefill: per layer the new tokens' slot mapping, store, and
    varlen multi-query paged attention; attention FLOP/s against the bf16
    matrix-core peak (causal pairs x Hq x 4 D flops)."""
    import torch

    import paged_kv_decode_store_amd as pkv
    from workloads.varlen import (varlen_attended_pairs, varlen_by_name, varlen_layer_inputs,
                                  varlen_tables)

    w = varlen_by_name(args.varlen)
    L = args.layers or w.num_layers
    Hq, Hkv, D, bs = w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    tables, cu_q, cu_k, nb = varlen_tables(w)
    T = int(cu_q[-1])
    mq, mk = int(np.diff(cu_q).max()), int(np.diff(cu_k).max())
    dev = torch.device("cuda")

    def u16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    td = torch.from_numpy(tables).to(dev)
    cq, ck = torch.from_numpy(cu_q).to(dev), torch.from_numpy(cu_k).to(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    kp = [torch.randn((nb, bs, Hkv, D), generator=gen, device=dev, dtype=torch.bfloat16)
          for _ in range(L)]
    vp = [torch.randn((nb, bs, Hkv, D), generator=gen, device=dev, dtype=torch.bfloat16)
          for _ in range(L)]
    lay = [varlen_layer_inputs(w, l) for l in range(L)]
    q = [u16(x[0]) for x in lay]
    kn = [u16(x[1]) for x in lay]
    vn = [u16(x[2]) for x in lay]
    slots = torch.empty(T, dtype=torch.int32, device=dev)
    out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=dev)
    B = len(w.lens_new)
    split = pkv.varlen_split_tokens(B, Hq, Hkv, mq, mk, args.split)
    need = pkv.varlen_workspace_bytes(T, B, Hq, Hkv, D, mq, mk, args.split)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    log(f"[bench] varlen {w.name}: {B} sequences, {T} new tokens, L={L}, split {split} "
        f"({'partials + merge' if need else 'one split'})")

    def step():
        pkv.varlen_slot_mapping(td, cq, ck, mq, bs, T, out=slots)
        for l in range(L):
            pkv.kv_store(kp[l], vp[l], kn[l], vn[l], slots)
            pkv.varlen_paged_attention(q[l], kp[l], vp[l], td, cq, ck, mq, mk,
                                       split_tokens=args.split, out=out, workspace=ws)

    def attn_only():
        for l in range(L):
            pkv.varlen_paged_attention(q[l], kp[l], vp[l], td, cq, ck, mq, mk,
                                       split_tokens=args.split, out=out, workspace=ws)

    def graph_ms(fn):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    step_ms = graph_ms(step)
    attn_us = 1e3 * graph_ms(attn_only) / L
    pairs = varlen_attended_pairs(w)
    flops = pairs * Hq * 4 * D
    tflops = flops / (attn_us * 1e-6) / 1e12
    kv_bytes = int(cu_k[-1]) * Hkv * D * 4
    io_bytes = kv_bytes + 2 * T * Hq * D * 2
    res = {
        "metric": "varlen paged attention TFLOP/s (chunked prefill)",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {len(w.lens_new)} sequences, new tokens "
                   f"{list(w.lens_new)} after cached {list(w.lens_cached)}, GQA {Hq}/{Hkv}, "
                   f"head_dim {D}, block {bs}, {L} layers",
                   "causal_pairs_per_head": pairs, "split_tokens": split,
                   "merge_step": bool(need)},
        "attention_us_per_layer": round(attn_us, 3),
        "attention_GBps": round(io_bytes / (attn_us * 1e-6) / 1e9, 1),
        "roofline": {"kernel": f"varlen_attention_kernel<{D}>", "bound": "mfma",
                     "achieved": round(tflops, 2), "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": round(tflops / 2500.0, 4), "flops_per_launch": flops,
                     "avg_launch_us": round(attn_us, 3), "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(res), flush=True)


def partial_kernel_name(cfg, D, fused, cascade):
    """Name of the partial-step kernel the library runs for this workload."""
    if cascade:
        return "cascade: decode_partial_mfma_kernel (prefix) + tail partial kernel + reduce"
    f = "true" if fused else "false"
    if cfg.group >= 3:  # the library's matrix-core threshold
        return f"decode_partial_mfma_kernel<{D}, {f}, 0>"  # mode 0: the decode step
    g = max(x for x in range(1, 9) if cfg.group % x == 0)
    return f"decode_partial_kernel<{D}, {g}, {f}>"


def stream_read_ceiling(dev, nbytes=1 << 31, launches=10):
    """Achieved rate of the library's streaming-read probe (16-byte
    non-temporal loads, 16 workgroups per CU, each over a contiguous share)
    over a fresh buffer far larger than the caches, timed with HIP events on
    the current stream."""
    import torch

    import paged_kv_decode_store_amd as pkv

    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(64, dtype=torch.int32, device=dev)
    for _ in range(2):
        pkv.probe_stream_read(buf, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(launches):
        pkv.probe_stream_read(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / launches
    del buf
    return {"GBps": round(nbytes / (us * 1e-6) / 1e9, 1), "bytes": nbytes, "us_per_launch":
            round(us, 2), "launches": launches,
            "how": "pkv_probe_stream_read: 16-byte non-temporal loads, each of 16 "
                   "workgroups of 256 threads per CU over a contiguous share, 8 loads in "
                   "flight per thread, HIP events"}


def read_traffic(name, fused, mfma):
    """Measured HBM bytes per launch of the partial kernel, from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source."""
    import hashlib

    tag = "fused" if fused else "plain"
    path = os.path.join(ROOT, "profiles", f"decode_partial_{tag}_{name}_counters.txt")
    src = os.path.join(ROOT, "paged_kv_decode_store_amd", "csrc",
                       "decode_attention_mfma.hip" if mfma else "decode_attention.hip")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            a, b = line.split(":", 1)
            kv[a.strip()] = b.strip()
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    if kv.get("kernel_source_sha256_16") != sha or "traffic_bytes_per_launch" not in kv:
        return None
    return int(float(kv["traffic_bytes_per_launch"]))


def host_description():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(),
            "usable_cpus": len(os.sched_getaffinity(0))}


def cpu_baseline(cfg, inp, kpool, vpool, seconds, threads):
    """The oracle as it stands on the host: attention of layer 0 over whole
    rows (pools copied back from the device), rows handed out to `threads`
    host threads (the C oracle runs outside the interpreter lock), repeated
    until about `seconds` of wall time; then a single-threaded run of a
    quarter of that.  Expressed in the same GB/s unit as `value`."""
    import threading

    import oracle
    import torch

    kh = kpool.view(torch.int16).cpu().numpy().view(np.uint16)
    vh = vpool.view(torch.int16).cpu().numpy().view(np.uint16)
    n, t = inp.context_lens, inp.block_tables
    q = inp.q[0]
    per_row = n.astype(np.int64) * cfg.num_kv_heads * cfg.head_dim * 4 + 4 * cfg.num_q_heads * cfg.head_dim
    host = host_description()
    T = threads or min(16, host["usable_cpus"])

    def run(nthreads, secs):
        lock = threading.Lock()
        state = {"next": 0, "rows": 0, "bytes": 0}
        t0 = time.perf_counter()

        def worker():
            while time.perf_counter() - t0 < secs:
                with lock:
                    b = state["next"] % cfg.batch
                    state["next"] += 1
                oracle.decode_attention(q[b:b + 1], kh, vh, t[b:b + 1], n[b:b + 1])
                with lock:
                    state["rows"] += 1
                    state["bytes"] += int(per_row[b])

        ws = [threading.Thread(target=worker) for _ in range(nthreads)]
        for w in ws:
            w.start()
        for w in ws:
            w.join()
        return state["rows"], state["bytes"], time.perf_counter() - t0

    rows, nbytes, elapsed = run(T, seconds)
    rows1, nbytes1, elapsed1 = run(1, seconds / 4)
    log(f"[bench] cpu oracle: {rows} rows in {elapsed:.1f} s on {T} threads; "
        f"{rows1} rows in {elapsed1:.1f} s on 1 thread")
    return {"value": round(nbytes / elapsed / 1e9, 4), "unit": "GB/s", "cores": T,
            "kind": "oracle",
            "sample": f"layer 0 attention of {rows} rows (cycling over the {cfg.batch} rows, "
                      f"fp64 two-pass softmax), {elapsed:.1f} s on {T} host threads",
            "single_thread_value": round(nbytes1 / elapsed1 / 1e9, 4),
            "host": host}


if __name__ == "__main__":
    main()
