"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: slot writes and sampled ids bit-exact; attention within max-abs 1e-2
of the fp64 oracle.  Sizes: the five workloads in the launch configuration
the benchmark times, plus small ragged cases that span several 16-position
chunks, several splits and a ragged tail.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_store_amd as pkv
from workloads import CONFIGS, config_by_name, host_inputs
from workloads.device import device_pool
from workloads.generate import block_tables, bf16_bits_from_f32, context_lengths, sampling_params

from gpu_util import (ATTN_TOL, bf16_out_to_f64, compare_ids, dev_f32, dev_i32, dev_u16,
                      host_u16, oracle_heads, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _normal_bf16(rng, shape):
    return bf16_bits_from_f32(rng.standard_normal(size=shape, dtype=np.float32))


# ------------------------------------------------------------ slot mapping --

@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: c.name)
def test_slot_mapping_workloads(cfg):
    n = context_lengths(cfg)
    t, _ = block_tables(cfg, n)
    say(f"slot_mapping {cfg.name}")
    got = pkv.slot_mapping(dev_i32(t), dev_i32(n), cfg.block_size).cpu().numpy()
    torch.cuda.synchronize()
    assert np.array_equal(got, oracle.slot_mapping(t, n, cfg.block_size))


def test_slot_mapping_edges():
    t = np.array([[5, 10], [3, -1], [7, 8]], np.int32)
    n = np.array([300, 257, 0], np.int32)  # row 1's position 256 hits the -1 entry
    for bs in (16, 256):
        got = pkv.slot_mapping(dev_i32(t), dev_i32(n), bs).cpu().numpy()
        assert np.array_equal(got, oracle.slot_mapping(t, n, bs)), bs
    # past the end of the table
    got = pkv.slot_mapping(dev_i32(t), dev_i32(np.array([600, 1, 1], np.int32)), 256).cpu().numpy()
    assert got.tolist() == oracle.slot_mapping(t, np.array([600, 1, 1], np.int32), 256).tolist()
    assert got[0] == -1


# --------------------------------------------------------------- kv store --

@pytest.mark.parametrize("name", ["tiny", "grok", "clone"])
def test_kv_store_host_pools(name):
    cfg = config_by_name(name)
    inp = host_inputs(cfg, layers=(0,), sampler=False)
    slots = oracle.slot_mapping(inp.block_tables, inp.context_lens, cfg.block_size)
    kc, vc = dev_u16(inp.k_pool[0]), dev_u16(inp.v_pool[0])
    say(f"kv_store {name}")
    pkv.kv_store(kc, vc, dev_u16(inp.k_new[0]), dev_u16(inp.v_new[0]), dev_i32(slots))
    torch.cuda.synchronize()
    kref, vref = inp.k_pool[0].copy(), inp.v_pool[0].copy()
    assert oracle.kv_store(kref, vref, inp.k_new[0], inp.v_new[0], slots, cfg.block_size) == 0
    assert np.array_equal(host_u16(kc), kref)
    assert np.array_equal(host_u16(vc), vref)


@pytest.mark.parametrize("name", ["qwen3", "long"])
def test_kv_store_device_pools(name):
    """Pools filled on the device: the rows at the slots must equal the new
    K/V bit for bit, and no other pool byte may change."""
    cfg = config_by_name(name)
    inp = host_inputs(cfg, layers=(0,), pools=False, sampler=False)
    slots = oracle.slot_mapping(inp.block_tables, inp.context_lens, cfg.block_size)
    kc = device_pool(cfg, inp.num_blocks, "kpool", 0)
    vc = device_pool(cfg, inp.num_blocks, "vpool", 0)
    k0, v0 = kc.clone(), vc.clone()
    say(f"kv_store {name}")
    pkv.kv_store(kc, vc, dev_u16(inp.k_new[0]), dev_u16(inp.v_new[0]), dev_i32(slots))
    torch.cuda.synchronize()
    rows = kc.shape[0] * kc.shape[1]
    sl = torch.from_numpy(slots.astype(np.int64)).cuda()
    for pool, before, new in ((kc, k0, inp.k_new[0]), (vc, v0, inp.v_new[0])):
        flat = pool.view(rows, -1)
        assert np.array_equal(host_u16(flat[sl]).reshape(new.shape), new)
        keep = torch.ones(rows, dtype=torch.bool, device="cuda")
        keep[sl] = False
        assert torch.equal(flat[keep].view(torch.int16), before.view(rows, -1)[keep].view(torch.int16))


def test_kv_store_skips_negative_and_out_of_range_slots():
    rng = np.random.default_rng(3)
    nb, bs, hkv, d = 3, 16, 2, 64
    kp, vp = _normal_bf16(rng, (nb, bs, hkv, d)), _normal_bf16(rng, (nb, bs, hkv, d))
    kn, vn = _normal_bf16(rng, (4, hkv, d)), _normal_bf16(rng, (4, hkv, d))
    slots = np.array([-1, 47, nb * bs, 0], np.int32)
    kc, vc = dev_u16(kp), dev_u16(vp)
    pkv.kv_store(kc, vc, dev_u16(kn), dev_u16(vn), dev_i32(slots))
    torch.cuda.synchronize()
    kref, vref = kp.copy(), vp.copy()
    oracle.kv_store(kref, vref, kn, vn, slots, bs)
    assert np.array_equal(host_u16(kc), kref) and np.array_equal(host_u16(vc), vref)


# -------------------------------------------------------------- attention --

def _attention_case(rng, B, Hq, Hkv, D, bs, lens, split, spare=3, scale=0.0):
    lens = np.asarray(lens, np.int32)
    need = [(int(n) + bs - 1) // bs for n in lens]
    W = max(1, max(need))
    nb = sum(need) + spare
    perm = rng.permutation(nb).astype(np.int32)
    tables = np.full((B, W), -1, np.int32)
    pos = 0
    for b in range(B):
        tables[b, :need[b]] = perm[pos:pos + need[b]]
        pos += need[b]
    kp, vp = _normal_bf16(rng, (nb, bs, Hkv, D)), _normal_bf16(rng, (nb, bs, Hkv, D))
    q = _normal_bf16(rng, (B, Hq, D))
    maxlen = int(max(1, lens.max()))
    say(f"attention B={B} Hq={Hq} Hkv={Hkv} D={D} bs={bs} split={split} lens={lens.tolist()}")
    out = pkv.paged_decode_attention(dev_u16(q), dev_u16(kp), dev_u16(vp), dev_i32(tables),
                                     dev_i32(lens), maxlen, scale=scale, split_tokens=split)
    torch.cuda.synchronize()
    ref = oracle.decode_attention(q, kp, vp, tables, lens, scale)
    return bf16_out_to_f64(out), ref


RAGGED = [1, 15, 16, 17, 63, 64, 65, 200, 255, 256, 257, 700]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 4), (6, 2), (12, 3), (10, 2), (14, 2), (8, 1),
                                    (16, 1), (22, 2)])
def test_attention_ragged_group_sizes(D, Hq, Hkv):
    rng = np.random.default_rng(1000 + D + 7 * Hq + Hkv)
    got, ref = _attention_case(rng, len(RAGGED), Hq, Hkv, D, 16, RAGGED, split=128)
    err = np.abs(got - ref).max()
    assert err <= ATTN_TOL, err


@pytest.mark.parametrize("bs", [16, 32, 64, 256])
@pytest.mark.parametrize("split", [0, 64, 192, 1024])
def test_attention_block_sizes_and_splits(bs, split):
    rng = np.random.default_rng(2000 + bs + split)
    lens = [0, 1, 31, 33, 100, 513, 1300, 64]
    got, ref = _attention_case(rng, len(lens), 8, 2, 128, bs, lens, split=split)
    assert np.abs(got - ref).max() <= ATTN_TOL
    assert np.all(got[0] == 0.0)  # inactive row -> zero vector


def test_attention_explicit_scale_and_peaky_scores():
    rng = np.random.default_rng(77)
    got, ref = _attention_case(rng, 3, 4, 2, 128, 16, [5, 300, 2000], split=64, scale=0.5)
    assert np.abs(got - ref).max() <= ATTN_TOL


def _decode_step_host(cfg, inp, layer=0):
    """Slot mapping + store + attention on the GPU for one layer of host
    pools; returns (gpu out fp64, oracle out fp64)."""
    n, t = inp.context_lens, inp.block_tables
    kc, vc = dev_u16(inp.k_pool[layer]), dev_u16(inp.v_pool[layer])
    nd, td = dev_i32(n), dev_i32(t)
    slots = pkv.slot_mapping(td, nd, cfg.block_size)
    pkv.kv_store(kc, vc, dev_u16(inp.k_new[layer]), dev_u16(inp.v_new[layer]), slots)
    out = pkv.paged_decode_attention(dev_u16(inp.q[layer]), kc, vc, td, nd, int(n.max()))
    torch.cuda.synchronize()
    kref, vref = inp.k_pool[layer].copy(), inp.v_pool[layer].copy()
    s_ref = oracle.slot_mapping(t, n, cfg.block_size)
    oracle.kv_store(kref, vref, inp.k_new[layer], inp.v_new[layer], s_ref, cfg.block_size)
    ref = oracle.decode_attention(inp.q[layer], kref, vref, t, n)
    return bf16_out_to_f64(out), ref


@pytest.mark.parametrize("name", ["tiny", "grok", "clone"])
def test_decode_step_workloads_full(name):
    cfg = config_by_name(name)
    inp = host_inputs(cfg, layers=(0,), sampler=False)
    say(f"decode step {name}")
    got, ref = _decode_step_host(cfg, inp)
    err = np.abs(got - ref).max()
    say(f"  max abs err {err:.3e}")
    assert err <= ATTN_TOL


def _device_layer(cfg, inp, layer):
    kc = device_pool(cfg, inp.num_blocks, "kpool", layer)
    vc = device_pool(cfg, inp.num_blocks, "vpool", layer)
    return kc, vc


def test_decode_step_qwen3_full_layers():
    """The headline workload: two layers of device-filled pools, every
    (row, head) output checked against the oracle."""
    cfg = config_by_name("qwen3")
    inp = host_inputs(cfg, layers=(0, 27), pools=False, sampler=False)
    n, t = inp.context_lens, inp.block_tables
    nd, td = dev_i32(n), dev_i32(t)
    slots = pkv.slot_mapping(td, nd, cfg.block_size)
    for li, layer in enumerate(inp.layers):
        say(f"decode step qwen3 layer {layer}")
        kc, vc = _device_layer(cfg, inp, layer)
        pkv.kv_store(kc, vc, dev_u16(inp.k_new[li]), dev_u16(inp.v_new[li]), slots)
        out = pkv.paged_decode_attention(dev_u16(inp.q[li]), kc, vc, td, nd, int(n.max()))
        torch.cuda.synchronize()
        kh, vh = host_u16(kc), host_u16(vc)  # pools after the store
        ref = oracle.decode_attention(inp.q[li], kh, vh, t, n)
        err = np.abs(bf16_out_to_f64(out) - ref).max()
        say(f"  max abs err {err:.3e}")
        assert err <= ATTN_TOL
        del kc, vc, kh, vh


def test_decode_step_long_sampled_heads():
    """Long-context split-KV workload at full size (matrix-core kernel, KV
    head rotated by split index); the threaded oracle checks two query
    heads of every KV head of every row (the first and last of its group on
    even rows, two middle ones on odd rows), which covers every split of
    every (row, KV head)."""
    cfg = config_by_name("long")
    inp = host_inputs(cfg, layers=(0,), pools=False, sampler=False)
    n, t = inp.context_lens, inp.block_tables
    nd, td = dev_i32(n), dev_i32(t)
    kc, vc = _device_layer(cfg, inp, 0)
    say("decode step long")
    slots = pkv.slot_mapping(td, nd, cfg.block_size)
    pkv.kv_store(kc, vc, dev_u16(inp.k_new[0]), dev_u16(inp.v_new[0]), slots)
    out = pkv.paged_decode_attention(dev_u16(inp.q[0]), kc, vc, td, nd, int(n.max()))
    torch.cuda.synchronize()
    got = bf16_out_to_f64(out)
    kh, vh = host_u16(kc), host_u16(vc)
    g = cfg.group
    pairs = []
    for b in range(cfg.batch):
        inner = (0, g - 1) if b % 2 == 0 else (g // 2 - 1, g // 2)
        pairs += [(b, kvh * g + i) for kvh in range(cfg.num_kv_heads) for i in inner]
    ref = oracle_heads(inp.q[0], kh, vh, t, n, pairs, g)
    worst = max(float(np.abs(got[b, h] - ref[(b, h)]).max()) for b, h in pairs)
    say(f"  max abs err {worst:.3e} over {len(pairs)} (row, head) pairs")
    assert worst <= ATTN_TOL


# ---------------------------------------------------------------- sampler --

def _sample_and_compare(z, g, t, p, k):
    ids = pkv.sample_next_token(dev_f32(z), dev_f32(g), dev_f32(t), dev_f32(p),
                                dev_i32(k)).cpu().numpy()
    torch.cuda.synchronize()
    ref, infos = oracle.sample(z, g, t, p, k)
    bad, amb = compare_ids(ids, ref, infos)
    return bad, amb, infos


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: c.name)
def test_sampler_workloads(cfg):
    inp = host_inputs(cfg, layers=(), pools=False)
    t, p, k = sampling_params(cfg)
    say(f"sampler {cfg.name}")
    bad, amb, infos = _sample_and_compare(inp.logits, inp.gumbel, t, p, k)
    say(f"  ambiguous rows {amb}, kept sizes {[i.kept for i in infos[:8]]}")
    assert not bad, bad
    assert amb == 0   # every workload row bit-exact, none excused


def test_sampler_mixed_rows_and_edges():
    rng = np.random.default_rng(55)
    B, V = 24, 50000  # V not a multiple of any chunk size
    z = (rng.standard_normal((B, V), dtype=np.float32) * 3).astype(np.float32)
    g = rng.gumbel(size=(B, V)).astype(np.float32)
    t = np.array([0.0, 0.7, 1.0, 1.3, -1.0, 0.01] * 4, np.float32)
    p = np.array([1.0, 0.9, 0.5, 0.0, 0.95, 0.3, 1.0, 0.99] * 3, np.float32)
    k = np.array([0, 0, 50, 1, V, 3, 1000, 0, 20, 0, 0, 7] * 2, np.int32)
    # exact ties: row 2 and 8 get repeated values around their k-th value
    z[2, :200] = 5.0
    z[8, 1000:1100] = 4.0
    z[8, 10] = 9.0
    bad, amb, _ = _sample_and_compare(z, g, t, p, k)
    assert not bad, bad
    assert amb == 0


def test_sampler_filters_follow_each_rows_settings():
    """Each row's own top_k and top_p decide its filters: k <= 0 or k >= V
    and p >= 1 turn a filter off for that row only, next to rows that use
    it, in one call."""
    rng = np.random.default_rng(56)
    B, V = 10, 9000
    z = (rng.standard_normal((B, V), dtype=np.float32) * 2).astype(np.float32)
    g = rng.gumbel(size=(B, V)).astype(np.float32)
    t = np.full(B, 0.9, np.float32)
    p = np.array([0.5, 1.0, 1.5, 0.5, 1.0, 0.5, 0.999, 1.0, 0.5, 0.0], np.float32)
    k = np.array([10, 10, 0, 0, -3, V, V + 5, 0, 1, 10], np.int32)
    bad, amb, infos = _sample_and_compare(z, g, t, p, k)
    assert not bad and amb == 0, bad
    assert [i.kept for i in infos[1:3]] == [10, V]    # top-k alone; nothing


def test_sampler_tiny_vocab_and_single_row():
    rng = np.random.default_rng(57)
    for V in (1, 2, 7, 1024, 1025):
        z = rng.standard_normal((1, V), dtype=np.float32)
        g = rng.gumbel(size=(1, V)).astype(np.float32)
        for (t, p, k) in ((1.0, 1.0, 0), (0.5, 0.6, 0), (1.0, 1.0, 2), (0.0, 1.0, 0)):
            bad, amb, _ = _sample_and_compare(z, g, np.array([t], np.float32),
                                              np.array([p], np.float32), np.array([k], np.int32))
            assert not bad, (V, t, p, k, bad)


def test_sampler_top_k_ties_across_chunks():
    """Many equal logits spread over several chunks: the kept ties must be
    the lowest indices, across chunk boundaries."""
    B, V = 4, 40000
    z = np.zeros((B, V), np.float32)
    z[:, ::7] = 1.0            # 5715 equal maxima per row
    g = np.random.default_rng(58).gumbel(size=(B, V)).astype(np.float32)
    t = np.ones(B, np.float32)
    p = np.ones(B, np.float32)
    k = np.array([1, 100, 3000, 5715], np.int32)
    bad, amb, infos = _sample_and_compare(z, g, t, p, k)
    assert not bad
    assert [i.kept for i in infos] == k.tolist()


# ------------------------------------------------ fused store + attention --

def _fused_case(rng, B, Hq, Hkv, D, bs, lens, split, spare=3):
    lens = np.asarray(lens, np.int32)
    need = [(int(n) + bs - 1) // bs for n in lens]
    W = max(1, max(need))
    nb = sum(need) + spare
    perm = rng.permutation(nb).astype(np.int32)
    tables = np.full((B, W), -1, np.int32)
    pos = 0
    for b in range(B):
        tables[b, :need[b]] = perm[pos:pos + need[b]]
        pos += need[b]
    kp, vp = _normal_bf16(rng, (nb, bs, Hkv, D)), _normal_bf16(rng, (nb, bs, Hkv, D))
    kn, vn = _normal_bf16(rng, (B, Hkv, D)), _normal_bf16(rng, (B, Hkv, D))
    q = _normal_bf16(rng, (B, Hq, D))
    maxlen = int(max(1, lens.max()))
    say(f"fused B={B} Hq={Hq} Hkv={Hkv} D={D} bs={bs} split={split} lens={lens.tolist()}")
    kc, vc = dev_u16(kp), dev_u16(vp)
    out = pkv.paged_decode_attention_store(dev_u16(q), kc, vc, dev_u16(kn), dev_u16(vn),
                                           dev_i32(tables), dev_i32(lens), maxlen,
                                           split_tokens=split)
    torch.cuda.synchronize()
    kref, vref = kp.copy(), vp.copy()
    slots = oracle.slot_mapping(tables, lens, bs)
    oracle.kv_store(kref, vref, kn, vn, slots, bs)
    ref = oracle.decode_attention(q, kref, vref, tables, lens)
    return bf16_out_to_f64(out), ref, host_u16(kc), host_u16(vc), kref, vref


@pytest.mark.parametrize("D,Hq,Hkv,bs,split", [
    (128, 16, 8, 256, 0), (128, 8, 2, 16, 64), (64, 16, 16, 32, 128), (128, 16, 1, 16, 64),
    (128, 22, 2, 64, 192), (64, 12, 4, 16, 0), (128, 48, 8, 256, 512)])
def test_fused_store_attention_matches_store_then_attend(D, Hq, Hkv, bs, split):
    """Ragged rows including n = 0, n = 1, new tokens at the first and last
    position of a block and of a 16-position chunk."""
    rng = np.random.default_rng(3000 + D + Hq + bs + split)
    lens = [0, 1, 2, 16, 17, 32, 33, bs, bs + 1, 2 * bs - 1, 700, 1025]
    got, ref, kh, vh, kref, vref = _fused_case(rng, len(lens), Hq, Hkv, D, bs, lens, split)
    assert np.array_equal(kh, kref) and np.array_equal(vh, vref)
    err = np.abs(got - ref).max()
    assert err <= ATTN_TOL, err
    assert np.all(got[0] == 0.0)


@pytest.mark.parametrize("name", ["tiny", "grok", "clone"])
def test_fused_decode_step_workloads_full(name):
    cfg = config_by_name(name)
    inp = host_inputs(cfg, layers=(0,), sampler=False)
    n, t = inp.context_lens, inp.block_tables
    kc, vc = dev_u16(inp.k_pool[0]), dev_u16(inp.v_pool[0])
    say(f"fused decode step {name}")
    out = pkv.paged_decode_attention_store(dev_u16(inp.q[0]), kc, vc, dev_u16(inp.k_new[0]),
                                           dev_u16(inp.v_new[0]), dev_i32(t), dev_i32(n),
                                           int(n.max()))
    torch.cuda.synchronize()
    kref, vref = inp.k_pool[0].copy(), inp.v_pool[0].copy()
    oracle.kv_store(kref, vref, inp.k_new[0], inp.v_new[0],
                    oracle.slot_mapping(t, n, cfg.block_size), cfg.block_size)
    assert np.array_equal(host_u16(kc), kref) and np.array_equal(host_u16(vc), vref)
    ref = oracle.decode_attention(inp.q[0], kref, vref, t, n)
    err = np.abs(bf16_out_to_f64(out) - ref).max()
    say(f"  max abs err {err:.3e}")
    assert err <= ATTN_TOL


def test_fused_decode_step_qwen3_layer():
    cfg = config_by_name("qwen3")
    inp = host_inputs(cfg, layers=(5,), pools=False, sampler=False)
    n, t = inp.context_lens, inp.block_tables
    kc, vc = _device_layer(cfg, inp, 5)
    k0, v0 = host_u16(kc), host_u16(vc)
    say("fused decode step qwen3 layer 5")
    out = pkv.paged_decode_attention_store(dev_u16(inp.q[0]), kc, vc, dev_u16(inp.k_new[0]),
                                           dev_u16(inp.v_new[0]), dev_i32(t), dev_i32(n),
                                           int(n.max()))
    torch.cuda.synchronize()
    kref, vref = k0, v0
    oracle.kv_store(kref, vref, inp.k_new[0], inp.v_new[0],
                    oracle.slot_mapping(t, n, cfg.block_size), cfg.block_size)
    assert np.array_equal(host_u16(kc), kref) and np.array_equal(host_u16(vc), vref)
    ref = oracle.decode_attention(inp.q[0], kref, vref, t, n)
    err = np.abs(bf16_out_to_f64(out) - ref).max()
    say(f"  max abs err {err:.3e}")
    assert err <= ATTN_TOL


# ------------------------------------------- sampler: threshold-bin paths --

def test_sampler_nucleus_threshold_bin_overflow():
    """More equal (or nearly equal) logits in the threshold bin than the
    candidate list holds: the cut is found by rescanning the row."""
    rng = np.random.default_rng(60)
    B, V = 4, 20000
    z = rng.standard_normal((B, V), dtype=np.float32)
    z[0] = 0.0                                   # all equal: every token kept
    z[1, :6000] = 3.0                            # 6000 tied maxima
    z[2] = (rng.integers(0, 3, V) * 1e-3).astype(np.float32)   # 3 values inside one bin
    g = rng.gumbel(size=(B, V)).astype(np.float32)
    t = np.ones(B, np.float32)
    p = np.array([0.5, 0.3, 0.7, 0.9], np.float32)
    k = np.zeros(B, np.int32)
    bad, amb, infos = _sample_and_compare(z, g, t, p, k)
    assert not bad, bad
    assert infos[0].kept == V and infos[1].kept >= 6000


def test_sampler_top_k_in_catch_all_bin_and_wide_spread():
    """Logits spread over thousands of units: most tokens sit in the last
    value bin; top-k ranks deep inside it and a nucleus near the top."""
    rng = np.random.default_rng(61)
    B, V = 4, 30000
    z = (rng.standard_normal((B, V), dtype=np.float32) * 500).astype(np.float32)
    g = rng.gumbel(size=(B, V)).astype(np.float32)
    t = np.array([1.0, 1.0, 0.01, 3.0], np.float32)
    p = np.array([1.0, 1.0, 0.9, 0.99], np.float32)
    k = np.array([V - 7, 25000, 0, 0], np.int32)
    bad, amb, _ = _sample_and_compare(z, g, t, p, k)
    assert not bad, bad


def test_sampler_top_k_then_nucleus_rounds():
    """Top-k then nucleus on the top-k set: the nucleus cut inside the top-k
    threshold bin, above it (a second round), and with overflowing ties."""
    rng = np.random.default_rng(62)
    B, V = 6, 40000
    z = (rng.standard_normal((B, V), dtype=np.float32) * 2).astype(np.float32)
    z[1, 123] = 30.0              # one dominant token: nucleus = {123}, far above the k bin
    z[2, :5000] = 6.0             # 5000 ties around the k-th value (overflow)
    z[3, 10:20] = 8.0
    z[3, 20:30] = 7.99            # nucleus cut among near-equal values
    g = rng.gumbel(size=(B, V)).astype(np.float32)
    t = np.array([1.0, 1.0, 1.0, 0.5, 0.8, 1.2], np.float32)
    p = np.array([0.9, 0.5, 0.6, 0.95, 0.3, 0.999], np.float32)
    k = np.array([500, 3000, 4500, 25, 2, 39000], np.int32)
    bad, amb, _ = _sample_and_compare(z, g, t, p, k)
    assert not bad, bad
    assert amb == 0


@pytest.mark.parametrize("seed", [63, 64, 65])
def test_sampler_random_mixed_settings(seed):
    """Random per-row settings over a mid-size batch, both filters enabled."""
    rng = np.random.default_rng(seed)
    B, V = 32, 50000
    z = (rng.standard_normal((B, V), dtype=np.float32) * rng.uniform(0.5, 6, (B, 1))).astype(np.float32)
    g = rng.gumbel(size=(B, V)).astype(np.float32)
    t = rng.choice([0.0, 0.3, 0.7, 1.0, 1.5], B).astype(np.float32)
    p = rng.choice([0.0, 0.2, 0.5, 0.9, 0.95, 1.0], B).astype(np.float32)
    k = rng.choice([0, 1, 10, 50, 1000, 20000], B).astype(np.int32)
    bad, amb, _ = _sample_and_compare(z, g, t, p, k)
    assert not bad, bad
    assert amb <= 1


def test_sampler_subnormal_scaled_logits():
    """Scaled logits z / T in and around the fp32 subnormal range (where the
    kernels divide instead of rounding a double product), huge and tiny
    temperatures, and many equal scaled values (ties go to the lowest
    index)."""
    rng = np.random.default_rng(61)
    B, V = 6, 20000
    tiny = np.float32(2.0 ** -149)
    z = np.empty((B, V), np.float32)
    z[0] = rng.integers(-2000, 2000, V).astype(np.float32) * tiny
    z[1] = rng.integers(-50, 50, V).astype(np.float32) * tiny
    z[2] = rng.standard_normal(V, dtype=np.float32)
    z[3] = rng.standard_normal(V, dtype=np.float32) * np.float32(1e-38)
    z[4] = rng.standard_normal(V, dtype=np.float32) * 3
    z[4, ::3] = rng.integers(-9, 9, len(z[4, ::3])).astype(np.float32) * tiny
    z[5] = rng.standard_normal(V, dtype=np.float32)
    g = rng.gumbel(size=(B, V)).astype(np.float32)
    t = np.array([10.0, 6.0, 3e38, 0.5, 10.0, 1e-30], np.float32)
    p = np.array([1.0, 1.0, 1.0, 1.0, 0.95, 1.0], np.float32)
    k = np.array([50, 100, 1000, 10, 0, 0], np.int32)
    bad, amb, infos = _sample_and_compare(z, g, t, p, k)
    assert not bad, bad
    assert [i.kept for i in infos[:4]] == k[:4].tolist()


@pytest.mark.parametrize("B,V", [(3, 1 << 24), (1, (1 << 24) - 3)])
def test_sampler_maximum_vocab(B, V):
    """The largest supported vocabulary (2^24) and an odd one just below it
    (single-float loads): thousands of chunks per row, more than the per-row
    kernels have threads, so their loops over the chunks' maxima and best
    keys run several rounds; nucleus, top-k and top-k then nucleus rows."""
    rng = np.random.default_rng(77 + B)
    z = (rng.standard_normal((B, V), dtype=np.float32) * 3).astype(np.float32)
    g = rng.gumbel(size=(B, V)).astype(np.float32)
    t = np.array([0.8, 1.0, 0.5][:B], np.float32)
    p = np.array([0.95, 1.0, 0.9][:B], np.float32)
    k = np.array([0, 50, 1000][:B], np.int32)
    z[-1, V - 1] = 14.0           # a high logit at the very end of the last row
    say(f"sampler B={B} V={V}")
    bad, amb, infos = _sample_and_compare(z, g, t, p, k)
    assert not bad, bad
    assert amb == 0


@pytest.mark.parametrize("n", [1, 16, 17, 63, 64, 65, 200, 256, 257, 300])
def test_sampler_cut_bin_sizes_and_ties(n):
    """Rows whose cut bin (1/32 of a unit below the row max) holds exactly n
    tokens, with pairs of tied values among them: up to 16 are resolved by
    one wave directly, up to 256 by one wave through value sub-ranges, more
    by the whole workgroup.  One top-k row (rank in the middle of the bin
    and on a tie) and one nucleus row per size; p sits halfway between two
    strictly-greater-mass levels, so no row is near a boundary."""
    rng = np.random.default_rng(7000 + n)
    V = 40000
    rows, ks, ps = [], [], []
    for kind in ("topk", "topk_tie", "nucleus"):
        z = np.minimum(rng.standard_normal(V), 4.0).astype(np.float32)
        idx = rng.choice(V, n + 1, replace=False)
        z[idx[0]] = 10.0                                     # the row max
        u = rng.uniform(0.05, 0.95, n)
        u[1::2] = u[0::2][:n // 2]                           # pairs of equal values
        z[idx[1:]] = (10.0 - (10.0 + u) / 32.0).astype(np.float32)   # all in bin 10
        rows.append(z)
        vals = np.sort(z[idx[1:]].astype(np.float64))[::-1]
        if kind == "topk":
            ks.append(1 + max(1, n // 2)); ps.append(1.0)
        elif kind == "topk_tie":
            j = int(np.flatnonzero(vals[:-1] == vals[1:])[0]) if n > 1 else 0
            ks.append(1 + j + 1); ps.append(1.0)             # rank on the first of a tie pair
        else:
            s64 = z.astype(np.float64)
            Z = np.exp(s64 - 10.0).sum()
            distinct = np.unique(vals)[::-1]                 # descending distinct values
            above = [1.0 + np.exp(vals[vals > v] - 10.0).sum() for v in distinct]
            j = len(distinct) // 2
            hi = above[j + 1] if j + 1 < len(above) else above[j] + np.exp(distinct[j] - 10.0)
            ks.append(0); ps.append(float((above[j] + hi) / 2.0 / Z))
    z = np.stack(rows)
    B = z.shape[0]
    g = rng.gumbel(size=(B, V)).astype(np.float32)
    t = np.ones(B, np.float32)
    say(f"sampler cut bin of {n} tokens")
    bad, amb, infos = _sample_and_compare(z, g, t, np.array(ps, np.float32), np.array(ks, np.int32))
    assert not bad, bad
    assert amb == 0
