"""GPU parity of the sampler's vocabulary mask and extra outputs (drawn-token
probability, top-8 ids and probabilities) against the CPU oracle.

Bars: ids and top-8 ids bit-exact (the order is decided by the fp32 scaled
logits, identical on both sides); probabilities within 1e-5 relative of the
fp64 oracle (the GPU sums exp(s - max) in fp64 from fp32 terms).  Nucleus
rows whose cut lies within 1e-5 of a mass boundary may differ (reported as
ambiguous).
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_store_amd as pkv
from workloads import CONFIGS, host_inputs
from workloads.generate import sampling_params

from gpu_util import AMBIGUOUS_MARGIN, dev_f32, dev_i32, say

pytestmark = pytest.mark.gpu

PROB_RTOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _run(z, g, t, p, k, mask=None, mask_stride_pad=0):
    B, V = z.shape
    mdev = None
    if mask is not None:
        if mask_stride_pad:
            # a padded row stride (not a multiple of 4): the unaligned path
            buf = np.zeros((B, V + mask_stride_pad), np.uint8)
            buf[:, :V] = mask
            mdev = torch.from_numpy(buf).cuda()[:, :V]
        else:
            mdev = torch.from_numpy(np.ascontiguousarray(mask, np.uint8)).cuda()
    ids, prob, tid, tpr = pkv.sample_next_token_ex(dev_f32(z), dev_f32(g), dev_f32(t), dev_f32(p),
                                                   dev_i32(k), mask=mdev)
    plain_ids = pkv.sample_next_token_ex(dev_f32(z), dev_f32(g), dev_f32(t), dev_f32(p),
                                         dev_i32(k), mask=mdev, extras=False)
    torch.cuda.synchronize()
    out = (ids.cpu().numpy(), prob.cpu().numpy(), tid.cpu().numpy(), tpr.cpu().numpy())
    assert np.array_equal(out[0], plain_ids.cpu().numpy())
    return out


def _compare(z, g, t, p, k, mask=None, **kw):
    B, V = z.shape
    ids, prob, tid, tpr = _run(z, g, t, p, k, mask, **kw)
    bad, amb = [], 0
    for b in range(B):
        info, x = oracle.sample_row_ex(z[b], g[b], t[b], p[b], k[b],
                                       None if mask is None else mask[b])
        ambiguous = info.topp_applied and info.margin <= AMBIGUOUS_MARGIN
        ok = (ids[b] == info.id and list(tid[b]) == list(x.top_ids)
              and abs(prob[b] - x.chosen_prob) <= PROB_RTOL * x.chosen_prob + 1e-30
              and np.all(np.abs(tpr[b] - np.array(x.top_probs)) <=
                         PROB_RTOL * np.array(x.top_probs) + 1e-30))
        if ok:
            continue
        if ambiguous:
            amb += 1
            continue
        bad.append((b, int(ids[b]), info.id, float(prob[b]), x.chosen_prob, list(tid[b]),
                    list(x.top_ids), list(tpr[b]), list(x.top_probs)))
    return bad, amb


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: c.name)
def test_extras_on_workloads_with_a_mask(cfg):
    inp = host_inputs(cfg, layers=(), pools=False)
    t, p, k = sampling_params(cfg)
    rng = np.random.default_rng(700 + cfg.index)
    mask = (rng.random(inp.logits.shape) < 0.9).astype(np.uint8)
    say(f"sampler extras {cfg.name} (masked)")
    bad, amb = _compare(inp.logits, inp.gumbel, t, p, k, mask)
    say(f"  ambiguous rows {amb}")
    assert not bad, bad[:2]
    assert amb == 0   # every workload row exact, none excused


@pytest.mark.parametrize("cfg", [CONFIGS[0], CONFIGS[1], CONFIGS[3]], ids=lambda c: c.name)
def test_extras_on_workloads_without_a_mask(cfg):
    inp = host_inputs(cfg, layers=(), pools=False)
    t, p, k = sampling_params(cfg)
    say(f"sampler extras {cfg.name}")
    bad, amb = _compare(inp.logits, inp.gumbel, t, p, k)
    assert not bad, bad[:2]
    assert amb == 0


def test_extras_edge_rows():
    rng = np.random.default_rng(71)
    B, V = 16, 30001                      # odd vocab: the single-float path
    z = (rng.standard_normal((B, V), dtype=np.float32) * 2).astype(np.float32)
    g = rng.gumbel(size=(B, V)).astype(np.float32)
    t = np.array([1.0, 0.0, 0.0, 0.8, 1.0, 1.2, 0.5, 1.0] * 2, np.float32)
    p = np.array([1.0, 1.0, 1.0, 0.0, 0.9, 1.0, 0.2, 0.6] * 2, np.float32)
    k = np.array([0, 0, 0, 0, 3, 5, 0, 40] * 2, np.int32)
    mask = np.ones((B, V), np.uint8)
    mask[0] = 0                           # every token forbidden: uniform
    z[1, [5, 900, 20000]] = 50.0          # greedy ties
    mask[2, z[2].argmax()] = 0            # greedy with its maximum forbidden
    mask[4, :100] = 0                     # top-k 3 (< 8: padded top list)
    mask[9, ::2] = 0
    z[10, :50] = 7.0                      # a block of equal values
    bad, amb = _compare(z, g, t, p, k, mask, mask_stride_pad=2)
    assert not bad, bad[:2]
    assert amb == 0


def test_extras_tiny_vocab_and_top_k_then_nucleus():
    rng = np.random.default_rng(72)
    for V in (1, 5, 8, 9):
        B = 6
        z = rng.standard_normal((B, V)).astype(np.float32)
        g = rng.gumbel(size=(B, V)).astype(np.float32)
        t = np.array([1.0, 0.0, 0.7, 1.0, 2.0, 1.0], np.float32)
        p = np.array([1.0, 1.0, 0.5, 0.9, 0.99, 0.3], np.float32)
        k = np.array([0, 0, 2, 3, 0, 4], np.int32)
        bad, amb = _compare(z, g, t, p, k)
        assert not bad, (V, bad[:2])
    # top-k then nucleus, including rows that need the second round
    B, V = 8, 20000
    z = (rng.standard_normal((B, V)) * 3).astype(np.float32)
    g = rng.gumbel(size=(B, V)).astype(np.float32)
    t = np.full(B, 0.9, np.float32)
    p = np.array([0.05, 0.2, 0.5, 0.9, 0.95, 0.99, 0.3, 0.7], np.float32)
    k = np.array([4000, 500, 50, 10, 3, 2000, 8, 100], np.int32)
    mask = (rng.random((B, V)) < 0.95).astype(np.uint8)
    bad, amb = _compare(z, g, t, p, k, mask)
    assert not bad, bad[:2]
    assert amb <= 1
