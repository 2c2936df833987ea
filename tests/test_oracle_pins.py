"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a worked
example printed on a page, a closed form, an invariant, a brute-force
computation organised differently, or a special case that reduces to a
library routine.  None of these tests needs a GPU.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from workloads import CONFIGS, bf16_bits_from_f32, f32_from_bf16_bits, host_inputs
from workloads.generate import block_tables, context_lengths

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(rng, shape, scale=1.0):
    return bf16_bits_from_f32(rng.standard_normal(size=shape).astype(np.float32) * np.float32(scale))


# ---------------------------------------------------------------- slots --

def test_slot_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "slot_example.json")))
    assert oracle.slot_for_position(g["block_table"], g["position"], g["block_size"]) == g["slot"]
    assert g["slot"] // g["block_size"] == g["physical_block"]
    assert g["slot"] % g["block_size"] == g["offset"]
    # the decode step writes the new token at position n - 1
    sm = oracle.slot_mapping(np.array([g["block_table"]], np.int32),
                             np.array([g["position"] + 1], np.int32), g["block_size"])
    assert sm.tolist() == [g["slot"]]


def test_block_bytes_golden():
    for c in json.load(open(os.path.join(GOLDEN, "block_bytes.json")))["cases"]:
        got = oracle.block_bytes(c["num_layers"], c["block_size"], c["num_kv_heads"],
                                 c["head_dim"], c["itemsize"])
        assert got == c["block_bytes"], c["source"]


@pytest.mark.parametrize("bs", [4, 16, 256])
def test_slot_map_is_a_bijection_onto_owned_blocks(bs):
    """Inverting slot -> (physical block, offset) through the table gives back
    every logical position exactly once, and rows never collide."""
    rng = np.random.default_rng(7)
    B, W = 5, 6
    nb = B * W + 3
    perm = rng.permutation(nb).astype(np.int32)
    tables = perm[:B * W].reshape(B, W)
    seen = set()
    for b in range(B):
        inv = {int(p): i for i, p in enumerate(tables[b])}
        for pos in range(W * bs):
            s = oracle.slot_for_position(tables[b], pos, bs)
            assert s >= 0 and s not in seen
            seen.add(s)
            logical = inv[s // bs]
            assert logical * bs + s % bs == pos
    # beyond the table, or an unset entry: no slot
    assert oracle.slot_for_position(tables[0], W * bs, bs) == -1
    assert oracle.slot_for_position(np.array([-1, 3], np.int32), 1, bs) == -1


def test_slot_mapping_inactive_rows():
    t = np.array([[3, 1], [0, 2]], np.int32)
    assert oracle.slot_mapping(t, np.array([0, 1], np.int32), 4).tolist() == [-1, 0]


# ---------------------------------------------------------------- store --

def test_store_writes_only_the_slots():
    rng = np.random.default_rng(1)
    nb, bs, hkv, d = 6, 4, 3, 8
    kc = _bf16(rng, (nb, bs, hkv, d))
    vc = _bf16(rng, (nb, bs, hkv, d))
    k0, v0 = kc.copy(), vc.copy()
    kn = _bf16(rng, (4, hkv, d))
    vn = _bf16(rng, (4, hkv, d))
    slots = np.array([5, -1, 23, 0], np.int32)
    assert oracle.kv_store(kc, vc, kn, vn, slots, bs) == 0
    fk = kc.reshape(nb * bs, hkv, d)
    fv = vc.reshape(nb * bs, hkv, d)
    for t, s in enumerate(slots):
        if s >= 0:
            assert np.array_equal(fk[s], kn[t]) and np.array_equal(fv[s], vn[t])
    mask = np.ones(nb * bs, bool)
    mask[[5, 23, 0]] = False
    assert np.array_equal(fk[mask], k0.reshape(nb * bs, hkv, d)[mask])
    assert np.array_equal(fv[mask], v0.reshape(nb * bs, hkv, d)[mask])
    # a slot past the pool is refused and writes nothing
    k1 = kc.copy()
    assert oracle.kv_store(kc, vc, kn[:1], vn[:1], np.array([nb * bs], np.int32), bs) == -1
    assert np.array_equal(kc, k1)


# ------------------------------------------------------------ attention --

def _causal_last_rows(qs, ks, vs, scale):
    """Full causal self-attention over a whole sequence, computed as one
    masked score matrix; returns every row.  qs [n, H, D], ks/vs [n, Hkv, D]
    (fp64).  GQA: head h reads KV head h // (H // Hkv)."""
    n, H, D = qs.shape
    g = H // ks.shape[1]
    out = np.zeros((n, H, D))
    mask = np.tril(np.ones((n, n), bool))
    for h in range(H):
        S = scale * (qs[:, h, :] @ ks[:, h // g, :].T)
        S = np.where(mask, S, -np.inf)
        P = np.exp(S - S.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        out[:, h, :] = P @ vs[:, h // g, :]
    return out


@pytest.mark.parametrize("n,H,Hkv", [(1, 2, 1), (7, 4, 2), (23, 3, 3), (40, 8, 2)])
def test_decode_row_equals_last_row_of_causal_attention(n, H, Hkv):
    """A decode step (store token n-1 at its slot, then attend over n cached
    positions) reproduces the last row of full causal attention over the
    whole sequence (KV-cache semantics)."""
    rng = np.random.default_rng(100 + n)
    D, bs = 8, 4
    qs = _bf16(rng, (n, H, D))
    ks = _bf16(rng, (n, Hkv, D))
    vs = _bf16(rng, (n, Hkv, D))
    need = (n + bs - 1) // bs
    nb = need + 3
    table = rng.permutation(nb)[:need].astype(np.int32)
    kc = _bf16(rng, (nb, bs, Hkv, D))  # junk everywhere first
    vc = _bf16(rng, (nb, bs, Hkv, D))
    # prefill positions 0..n-2 into the paged cache
    for j in range(n - 1):
        s = oracle.slot_for_position(table, j, bs)
        kc.reshape(-1, Hkv, D)[s] = ks[j]
        vc.reshape(-1, Hkv, D)[s] = vs[j]
    # decode step: slot of the new token, store, attend
    slots = oracle.slot_mapping(table[None, :], np.array([n], np.int32), bs)
    assert oracle.kv_store(kc, vc, ks[n - 1:n], vs[n - 1:n], slots, bs) == 0
    got = oracle.decode_attention(qs[n - 1:n], kc, vc, table[None, :], np.array([n], np.int32))
    ref = _causal_last_rows(f32_from_bf16_bits(qs).astype(np.float64),
                            f32_from_bf16_bits(ks).astype(np.float64),
                            f32_from_bf16_bits(vs).astype(np.float64), 1.0 / math.sqrt(D))
    np.testing.assert_allclose(got[0], ref[n - 1], rtol=0, atol=1e-12)


def test_paged_equals_contiguous_and_relabelling():
    """Paged gather over a random block permutation equals attention over the
    contiguous (B, T, H, D) cache; relabelling physical blocks changes
    nothing."""
    rng = np.random.default_rng(5)
    B, Hq, Hkv, D, bs = 3, 4, 2, 16, 8
    n = np.array([1, 13, 37], np.int32)
    T = 40
    kcont = _bf16(rng, (B, T, Hkv, D))
    vcont = _bf16(rng, (B, T, Hkv, D))
    q = _bf16(rng, (B, Hq, D))
    W = (T + bs - 1) // bs
    nb = B * W + 2
    perm = rng.permutation(nb).astype(np.int32)
    tables = perm[:B * W].reshape(B, W)
    kc = _bf16(rng, (nb, bs, Hkv, D))
    vc = _bf16(rng, (nb, bs, Hkv, D))
    for b in range(B):
        for j in range(T):
            s = oracle.slot_for_position(tables[b], j, bs)
            kc.reshape(-1, Hkv, D)[s] = kcont[b, j]
            vc.reshape(-1, Hkv, D)[s] = vcont[b, j]
    paged = oracle.decode_attention(q, kc, vc, tables, n)
    cont = oracle.contiguous_attention(q, kcont, vcont, n)
    np.testing.assert_allclose(paged, cont, rtol=0, atol=1e-14)
    # relabel: physical block p -> sigma(p)
    sigma = rng.permutation(nb).astype(np.int32)
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[sigma] = kc
    vc2[sigma] = vc
    relabelled = oracle.decode_attention(q, kc2, vc2, sigma[tables], n)
    np.testing.assert_allclose(relabelled, paged, rtol=0, atol=1e-14)


def test_attention_closed_forms():
    rng = np.random.default_rng(9)
    Hkv, D, bs = 2, 8, 4
    nb = 4
    kc = _bf16(rng, (nb, bs, Hkv, D))
    vc = _bf16(rng, (nb, bs, Hkv, D))
    q = _bf16(rng, (1, 2, D))
    table = np.array([[2, 0, 3]], np.int32)
    # n = 1: the only weight is 1, so o = V of position 0 exactly
    o1 = oracle.decode_attention(q, kc, vc, table, np.array([1], np.int32))
    for h in range(2):
        np.testing.assert_array_equal(o1[0, h], f32_from_bf16_bits(vc[2, 0, h]).astype(np.float64))
    # n = 0: inactive row -> zero vector
    o0 = oracle.decode_attention(q, kc, vc, table, np.array([0], np.int32))
    assert np.all(o0 == 0.0)
    # equal keys everywhere: uniform weights, o = mean of V rows
    kc_eq = kc.copy()
    kc_eq[:] = kc[0, 0]
    n = 11
    oe = oracle.decode_attention(q, kc_eq, vc, table, np.array([n], np.int32))
    rows = [f32_from_bf16_bits(vc.reshape(-1, Hkv, D)[oracle.slot_for_position(table[0], j, bs)])
            for j in range(n)]
    mean = np.mean(np.stack(rows).astype(np.float64), axis=0)
    np.testing.assert_allclose(oe[0], mean, rtol=0, atol=1e-13)
    # softmax is shift invariant: the same equal keys at a scale that puts
    # every score near 1e4 (exp overflows fp64 without subtracting the max)
    # still give the mean of V; and two distinct scores 1e4 apart give the V
    # of the larger one alone
    oe_big = oracle.decode_attention(q, kc_eq, vc, table, np.array([n], np.int32), scale=1e4)
    np.testing.assert_allclose(oe_big[0], mean, rtol=0, atol=1e-13)
    kc2 = np.zeros_like(kc)                       # score 0 at position 0
    one = bf16_bits_from_f32(np.ones(D, np.float32))
    kc2[0, 1] = one                               # position 1: q . 1 at slot 1
    q2 = np.broadcast_to(one, (1, 2, D)).copy()   # q . 1 = D = 8 > 0
    o2 = oracle.decode_attention(q2, kc2, vc, np.array([[0]], np.int32), np.array([2], np.int32),
                                 scale=1250.0)   # scores 0 and 1e4
    for h in range(2):
        np.testing.assert_array_equal(o2[0, h], f32_from_bf16_bits(vc[0, 1, h]).astype(np.float64))


def test_gqa_equals_mha_with_repeated_heads():
    rng = np.random.default_rng(11)
    B, Hq, Hkv, D, bs = 2, 6, 2, 8, 4
    g = Hq // Hkv
    nb = 8
    kc = _bf16(rng, (nb, bs, Hkv, D))
    vc = _bf16(rng, (nb, bs, Hkv, D))
    q = _bf16(rng, (B, Hq, D))
    tables = np.array([[1, 4, 6, 0], [7, 2, 3, 5]], np.int32)
    n = np.array([14, 9], np.int32)
    gqa = oracle.decode_attention(q, kc, vc, tables, n)
    mha = oracle.decode_attention(q, np.repeat(kc, g, axis=2), np.repeat(vc, g, axis=2), tables, n)
    np.testing.assert_array_equal(gqa, mha)


def test_lse_merge_of_partials_equals_unsplit():
    """The split-KV reduce rule: attention over disjoint token ranges,
    merged with weights exp(m_s - M) l_s, equals attention over the union.
    Partials are formed from per-range oracle outputs: o_s = attn over range
    s, l_s = sum exp(score - m_s)."""
    rng = np.random.default_rng(13)
    D, bs, n = 8, 4, 29
    kc = _bf16(rng, (8, bs, 1, D))
    vc = _bf16(rng, (8, bs, 1, D))
    q = _bf16(rng, (1, 1, D))
    table = rng.permutation(8).astype(np.int32)
    full = oracle.decode_attention(q, kc, vc, table[None], np.array([n], np.int32))[0, 0]
    scale = 1.0 / math.sqrt(D)
    qf = f32_from_bf16_bits(q[0, 0]).astype(np.float64)
    kflat = f32_from_bf16_bits(kc.reshape(-1, D)).astype(np.float64)
    slots = [oracle.slot_for_position(table, j, bs) for j in range(n)]
    for cuts in ([0, 29], [0, 4, 29], [0, 1, 8, 17, 28, 29]):
        ms, ls, os_ = [], [], []
        for a, b in zip(cuts[:-1], cuts[1:]):
            # a range [a, b) is attention of the positions a..b-1: shift the
            # table so that the oracle sees exactly those positions
            sc = np.array([scale * kflat[slots[j]] @ qf for j in range(a, b)])
            m = sc.max()
            ls.append(np.exp(sc - m).sum())
            ms.append(m)
            kc_r = np.stack([kc.reshape(-1, 1, D)[slots[j]] for j in range(a, b)])[None]
            vc_r = np.stack([vc.reshape(-1, 1, D)[slots[j]] for j in range(a, b)])[None]
            os_.append(oracle.contiguous_attention(q, kc_r, vc_r, np.array([b - a], np.int32))[0, 0])
        M = max(ms)
        wts = [math.exp(m - M) * l for m, l in zip(ms, ls)]
        merged = sum(w * o for w, o in zip(wts, os_)) / sum(wts)
        np.testing.assert_allclose(merged, full, rtol=0, atol=1e-13)


def test_attention_rejects_bad_block_id():
    rng = np.random.default_rng(3)
    kc = _bf16(rng, (2, 4, 1, 8))
    with pytest.raises(ValueError):
        oracle.decode_attention(_bf16(rng, (1, 1, 8)), kc, kc, np.array([[0, 5]], np.int32),
                                np.array([6], np.int32))


# --------------------------------------------------------------- sampler --

def test_greedy_is_argmax_lowest_index():
    rng = np.random.default_rng(21)
    z = rng.standard_normal(1000).astype(np.float32)
    g = rng.gumbel(size=1000).astype(np.float32)
    info = oracle.sample_row(z, g, 0.0, 0.9, 5)
    assert info.greedy == 1 and info.id == int(np.argmax(z))
    z2 = np.zeros(16, np.float32)
    z2[[3, 9]] = 2.0
    assert oracle.sample_row(z2, g[:16], 0.0, 1.0, 0).id == 3


def test_small_temperature_is_greedy_when_gap_dominates_noise():
    rng = np.random.default_rng(22)
    V = 4096
    for trial in range(20):
        z = rng.standard_normal(V).astype(np.float32) * 4
        g = rng.gumbel(size=V).astype(np.float32)
        srt = np.sort(z)
        T = np.float32(0.01)
        if (srt[-1] - srt[-2]) / T > g.max() - g.min() + 1:
            assert oracle.sample_row(z, g, T, 1.0, 0).id == int(np.argmax(z))


def test_plain_temperature_sampling_is_gumbel_argmax():
    """p = 1, k = 0 keeps all V; with T = 1 the draw is argmax(z + g)."""
    rng = np.random.default_rng(23)
    V = 5000
    z = rng.standard_normal(V).astype(np.float32)
    g = rng.gumbel(size=V).astype(np.float32)
    info = oracle.sample_row(z, g, 1.0, 1.0, 0)
    assert info.kept == V
    assert info.id == int(np.argmax(z + g))


def test_top_k_one_is_argmax_and_equal_logits_keep_lowest_indices():
    rng = np.random.default_rng(24)
    z = rng.standard_normal(300).astype(np.float32)
    g = rng.gumbel(size=300).astype(np.float32)
    assert oracle.sample_row(z, g, 0.7, 1.0, 1).id == int(np.argmax(z))
    flat = np.zeros(50, np.float32)
    info = oracle.sample_row(flat, g[:50], 1.0, 1.0, 3)
    assert info.kept == 3 and info.id == int(np.argmax(g[:3]))


def test_nucleus_closed_forms():
    g = np.random.default_rng(25).gumbel(size=64).astype(np.float32)
    # one dominant token holds more than p of the mass: nucleus of size 1
    z = np.zeros(64, np.float32)
    z[17] = 10.0
    info = oracle.sample_row(z, g, 1.0, 0.9, 0)
    assert info.kept == 1 and info.id == 17
    # uniform logits: every token has mass 1/V; the nucleus keeps all ties
    info = oracle.sample_row(np.zeros(64, np.float32), g, 1.0, 0.5, 0)
    assert info.kept == 64
    # p <= 0 keeps only the maxima; no mass is compared, so no rounding can
    # move that cut: its margin is infinite (never excused as ambiguous)
    z3 = np.arange(64, dtype=np.float32) % 7
    info = oracle.sample_row(z3, g, 1.0, 0.0, 0)
    assert info.kept == int(np.sum(z3 == z3.max()))
    assert info.margin == float("inf")


def test_temperature_applies_before_nucleus():
    """Two tokens: logits 0 and 1, p = 0.6.  At T = 1 the top token holds
    e/(1+e) = 0.731 > 0.6 -> nucleus {top}; at T = 4 it holds 0.562 < 0.6 ->
    both kept.  Filtering the unscaled logits would give {top} in both."""
    g = np.array([5.0, -5.0], np.float32)  # noise favours index 0
    z = np.array([0.0, 1.0], np.float32)
    assert oracle.sample_row(z, g, 1.0, 0.6, 0).kept == 1
    info = oracle.sample_row(z, g, 4.0, 0.6, 0)
    assert info.kept == 2 and info.id == 0


def _nucleus_by_definition(s, p):
    """Smallest group-prefix (descending distinct values) whose mass exceeds
    p, with exact rational arithmetic on rounded weights; returns the kept
    index set.  Weights are exp(s - max) rounded to 1e-12 as fractions."""
    w = [Fraction(round(math.exp(x - max(s)) * 1e12)) for x in s]
    Z = sum(w)
    vals = sorted(set(s), reverse=True)
    kept_vals = []
    mass = Fraction(0)
    for v in vals:
        kept_vals.append(v)
        mass += sum(wi for wi, x in zip(w, s) if x == v)
        if mass / Z > Fraction(p):
            break
    return {i for i, x in enumerate(s) if x in kept_vals}, mass / Z


def test_nucleus_page_rule_matches_definition_on_tiny_vocab():
    """The page's ascending-cumsum rule (sort ascending, cumsum of softmax,
    first index reaching 1 - p, keep >= that logit) equals the direct
    definition on small vocabularies, including ties."""
    rng = np.random.default_rng(26)
    checked = 0
    for trial in range(400):
        V = int(rng.integers(2, 11))
        s = (rng.integers(-4, 5, size=V) * 0.75).astype(np.float32)  # many ties
        p = float(np.float32(rng.uniform(0.05, 0.99)))
        info = oracle.sample_row(s, np.zeros(V, np.float32), 1.0, p, 0)
        if info.margin < 1e-9:
            continue
        kept_def, _ = _nucleus_by_definition([float(x) for x in s], p)
        kept_oracle = {i for i in range(V) if s[i] >= info.tau}
        assert kept_oracle == kept_def, (s, p)
        assert info.kept == len(kept_def)
        checked += 1
    assert checked > 300


def test_top_k_then_nucleus_takes_the_nucleus_of_the_top_k_set():
    """Runners chapter 8.3 masks to the top k, then filters by top-p: the
    nucleus is taken over the softmax of the kept k tokens.  z = [2, 1 x 9],
    T = 1, k = 2 keeps {0, 1} (the 1.0 tie goes to the lower index); over
    that set token 0 holds e/(e+1) = 0.731 > p = 0.5 of the mass, so the
    nucleus is {0} alone.  Over all ten tokens token 0 holds only
    e/(e+9) = 0.232, so a nucleus over the whole vocabulary would keep the
    1.0 group too, i.e. both tokens of the top-k set."""
    z = np.array([2.0] + [1.0] * 9, np.float32)
    g = np.array([-5.0, 5.0] + [0.0] * 8, np.float32)  # noise favours index 1
    info = oracle.sample_row(z, g, 1.0, 0.5, 2)
    assert info.kept == 1 and info.id == 0 and info.tau == 2.0
    # the same row with the top-k set's own mass boundary on the other side:
    # p = 0.75 > e/(e+1) needs both kept tokens
    info = oracle.sample_row(z, g, 1.0, 0.75, 2)
    assert info.kept == 2 and info.id == 1
    # closed form of the margin over the top-k set: the cut sits in the
    # group {2.0} whose strictly-below mass is 1/(e+1) and through-mass 1
    e = math.e
    target = 1.0 - float(np.float32(0.5))
    m_exact = min(target - 1 / (e + 1), 1.0 - target)
    info = oracle.sample_row(z, g, 1.0, 0.5, 2)
    assert abs(info.margin - m_exact) < 1e-12


def test_nucleus_margin_closed_forms():
    """margin = distance from the cut's target 1 - p to the nearer mass
    boundary of the threshold value's tie group (mass strictly below tau,
    mass up to and including tau), in normalised mass."""
    g0 = np.zeros(8, np.float32)
    # eight equal logits: masses 1/8 each; 1 - p = 0.3125 lies inside the
    # one tie group [0, 1], 3/8 of the way along the cumsum (its third
    # member reaches it first): distance 0.3125 to the lower edge 0, 0.6875
    # to the upper edge 1
    info = oracle.sample_row(np.zeros(8, np.float32), g0, 1.0, 0.6875, 0)
    assert info.kept == 8 and info.tau == 0.0
    assert info.margin == 0.3125
    # s = [1, 1, 1, 0, 0]: masses a = 1/(3e+2) for the zeros, b = e/(3e+2)
    # for the ones; ascending cumsum a, 2a, 2a+b, 2a+2b, 1.  1 - p at 2a +
    # 1.2 b is reached first at the second 1 (index 3), inside the group
    # {1} whose edges are 2a (below) and 1 (through).
    e = math.e
    a, b = 1 / (3 * e + 2), e / (3 * e + 2)
    p = np.float32(1.0 - (2 * a + 1.2 * b))
    target = 1.0 - float(p)
    s = np.array([1.0, 1.0, 1.0, 0.0, 0.0], np.float32)
    info = oracle.sample_row(s, np.zeros(5, np.float32), 1.0, p, 0)
    assert info.kept == 3 and info.tau == 1.0
    m1, m2 = target - 2 * a, 1.0 - target
    assert m1 < m2
    assert abs(info.margin - m1) < 1e-12
    # upper edge nearer: 1 - p at 1.25 a lies inside the group {0}, whose
    # edges are 0 and 2a; the nearer one is 2a, 0.75 a away
    p2 = np.float32(1.0 - 1.25 * a)
    target2 = 1.0 - float(p2)
    info = oracle.sample_row(s, np.zeros(5, np.float32), 1.0, p2, 0)
    assert info.kept == 5 and info.tau == 0.0
    assert abs(info.margin - min(target2 - 0.0, 2 * a - target2)) < 1e-12


def test_nucleus_margin_is_the_distance_to_a_change_of_the_kept_set():
    """What the margin means: moving p by 0.9 x margin either way keeps the
    kept set, while moving it 1.1 x margin towards the nearer boundary
    changes it.  Random small rows with ties; rows whose cut lies in the
    lowest or the highest kept value group are skipped: the lower edge of
    the lowest group (mass 0) and the upper edge of the highest (mass 1)
    cannot be crossed by any 0 < p < 1, so there the margin is only a
    conservative bound."""
    rng = np.random.default_rng(28)
    checked = 0
    for trial in range(1000):
        V = int(rng.integers(3, 12))
        s = (rng.integers(-3, 4, size=V) * 0.5).astype(np.float32)
        p = np.float32(rng.uniform(0.05, 0.95))
        k = int(rng.integers(0, V + 1)) if trial % 2 else 0
        base = oracle.sample_row(s, np.zeros(V, np.float32), 1.0, p, k)
        m = base.margin
        kept_vals = np.sort(s)[::-1][:k] if 0 < k < V else s
        if m < 1e-4 or base.tau in (kept_vals.min(), kept_vals.max()):
            continue
        for sign in (1.0, -1.0):
            q = np.float32(float(p) + sign * 0.9 * m)
            info = oracle.sample_row(s, np.zeros(V, np.float32), 1.0, q, k)
            assert info.kept == base.kept, (s, p, k, m, sign)
        changed = []
        for sign in (1.0, -1.0):
            q = np.float32(min(max(float(p) + sign * 1.1 * m, 1e-6), 1.0))
            info = oracle.sample_row(s, np.zeros(V, np.float32), 1.0, q, k)
            changed.append(info.kept != base.kept)
        assert any(changed), (s, p, k, m)
        checked += 1
    assert checked > 250


def test_sampled_distribution_matches_softmax_on_eligible_set():
    """Chi-square over 100000 Gumbel draws: ids follow softmax(z / T)
    renormalised on the eligible set (top-k then nucleus)."""
    rng = np.random.default_rng(27)
    V, N = 8, 100000
    z = np.array([2.0, 1.5, 1.0, 0.4, 0.0, -0.5, -1.0, -3.0], np.float32)
    T, p, k = np.float32(0.8), np.float32(0.9), 6
    g = rng.gumbel(size=(N, V)).astype(np.float32)
    ids, infos = oracle.sample(np.tile(z, (N, 1)), g, np.full(N, T, np.float32),
                               np.full(N, p, np.float32), np.full(N, k, np.int32))
    s = (z / T).astype(np.float64)
    order = np.argsort(-s, kind="stable")
    elig = np.zeros(V, bool)
    elig[order[:k]] = True
    w = np.where(elig, np.exp(s - s.max()), 0.0)
    w /= w.sum()
    # nucleus on the top-k set: smallest descending prefix with mass > p
    cum = 0.0
    nuc = np.zeros(V, bool)
    for i in order[:k]:
        nuc[i] = True
        cum += w[i]
        if cum > p:
            break
    probs = np.where(nuc, w, 0.0)
    probs /= probs.sum()
    assert infos[0].kept == nuc.sum()
    counts = np.bincount(ids, minlength=V)
    assert counts[~nuc].sum() == 0
    exp_ = probs[nuc] * N
    chi2 = float(np.sum((counts[nuc] - exp_) ** 2 / exp_))
    dof = int(nuc.sum()) - 1
    # 99.9% quantile of chi-square with <= 7 dof is < 24.4
    assert chi2 < 24.4, (chi2, dof, counts, exp_)


def test_gumbel_noise_moments():
    inp = host_inputs(CONFIGS[0], pools=False)
    g = inp.gumbel.astype(np.float64).ravel()
    assert abs(g.mean() - 0.5772156649) < 0.01
    assert abs(g.var() - math.pi ** 2 / 6) < 0.02


def test_workload_tables_are_consistent():
    """Every workload's block tables cover n_b positions with in-range,
    non-colliding blocks (except the clone workload's shared prefix)."""
    for cfg in CONFIGS:
        n = context_lengths(cfg)
        t, nb = block_tables(cfg, n)
        need = (n.astype(np.int64) + cfg.block_size - 1) // cfg.block_size
        owned = []
        for b in range(cfg.batch):
            row = t[b, :need[b]]
            assert np.all((row >= 0) & (row < nb))
            owned.append(row[cfg.clone_prefix_blocks:])
        allowned = np.concatenate(owned)
        assert len(set(allowned.tolist())) == len(allowned)


# ------------------------------------------- sampler mask and extra outputs --

def _softmax64(x):
    # scipy's softmax, the library routine the unfiltered case reduces to
    from scipy.special import softmax
    return softmax(np.asarray(x, np.float64))


def test_extras_without_filters_equal_library_softmax():
    """p = 1, k = 0, no mask: the drawn id's probability and the top 8 are
    those of softmax(z / T) (stable argsort for the order)."""
    rng = np.random.default_rng(91)
    V = 300
    z = (rng.standard_normal(V) * 2).astype(np.float32)
    z[[10, 11]] = z.max() + 1.0          # a tie at the top: lower index first
    g = rng.gumbel(size=V).astype(np.float32)
    T = np.float32(0.7)
    info, x = oracle.sample_row_ex(z, g, T, 1.0, 0)
    pr = _softmax64(z / T)
    assert abs(x.chosen_prob - pr[info.id]) < 1e-12
    order = np.argsort(-pr, kind="stable")[:8]
    assert list(x.top_ids) == order.tolist()
    assert np.allclose(list(x.top_probs), pr[order], rtol=1e-12, atol=0)
    assert x.top_ids[0] == 10 and x.top_ids[1] == 11


def test_mask_forbids_tokens_and_is_applied_after_temperature():
    rng = np.random.default_rng(92)
    V = 50
    z = rng.standard_normal(V).astype(np.float32)
    mask = np.zeros(V, np.uint8)
    mask[[3, 17, 40]] = 1
    for trial in range(200):
        g = rng.gumbel(size=V).astype(np.float32)
        info, x = oracle.sample_row_ex(z, g, 1.3, 1.0, 0, mask=mask)
        assert info.id in (3, 17, 40)
        assert x.top_ids[:3].__len__() == 3 and set(x.top_ids[:3]) == {3, 17, 40}
        assert all(p == 0.0 for p in x.top_probs[3:])
        assert abs(sum(x.top_probs) - 1.0) < 1e-12
    # the page divides by T first, then sets forbidden tokens to -1e10: with
    # T = 0.05 an allowed logit of -1e9 scales to -2e10, below the forbidden
    # tokens' -1e10, so a forbidden token (the lowest-index one) is drawn
    z2 = np.full(4, -1e9, np.float32)
    info, _ = oracle.sample_row_ex(z2, np.zeros(4, np.float32), 0.05, 1.0, 0,
                                   mask=np.array([1, 0, 1, 0], np.uint8))
    assert info.id == 1


def test_all_masked_row_is_uniform():
    V = 37
    z = np.linspace(-3, 3, V).astype(np.float32)
    g = np.random.default_rng(93).gumbel(size=V).astype(np.float32)
    info, x = oracle.sample_row_ex(z, g, 1.0, 1.0, 0, mask=np.zeros(V, np.uint8))
    # every key is fl32(-1e10 + g) == -1e10: a tie, lowest index
    assert info.id == 0
    assert abs(x.chosen_prob - 1.0 / V) < 1e-15
    assert list(x.top_ids) == list(range(8))


def test_extras_under_top_k_and_nucleus():
    z = np.array([0.5, 3.0, 2.0, -1.0, 2.0, 1.0, 0.0, -2.0, 1.5, 0.2], np.float32)
    g = np.zeros_like(z)
    # top-k 3: the kept set is {1, 2, 4} (2.0 tie: both kept, k = 3)
    info, x = oracle.sample_row_ex(z, g, 1.0, 1.0, 3)
    pr = _softmax64(z[[1, 2, 4]])
    assert list(x.top_ids[:3]) == [1, 2, 4]
    assert np.allclose(list(x.top_probs[:3]), pr, rtol=1e-12, atol=0)
    # then the lowest-index ids outside the kept set, probability 0
    assert list(x.top_ids[3:]) == [0, 3, 5, 6, 7]
    assert list(x.top_probs[3:]) == [0.0] * 5
    assert info.id == 1 and abs(x.chosen_prob - pr[0]) < 1e-12
    # nucleus p = 0.5 on the full set keeps the smallest prefix with mass
    # > 0.5, plus every value tied with its last one (here: 2.0 twice)
    full = _softmax64(z)
    order = np.argsort(-full, kind="stable")
    last = order[np.searchsorted(np.cumsum(full[order]), 0.5, side="right")]
    keep = np.nonzero(z >= z[last])[0]
    assert len(keep) == 3
    info, x = oracle.sample_row_ex(z, g, 1.0, 0.5, 0)
    assert info.kept == len(keep)
    pk = _softmax64(z[np.sort(keep)])
    got = dict(zip(x.top_ids[:len(keep)], x.top_probs[:len(keep)]))
    for i, p in zip(np.sort(keep), pk):
        assert abs(got[i] - p) < 1e-12


def test_greedy_extras_split_ties_and_respect_the_mask():
    z = np.array([1.0, 4.0, 2.0, 4.0, 4.0, 0.0], np.float32)
    info, x = oracle.sample_row_ex(z, np.zeros_like(z), 0.0, 1.0, 0)
    assert info.id == 1 and abs(x.chosen_prob - 1 / 3) < 1e-15
    assert list(x.top_ids[:3]) == [1, 3, 4] and list(x.top_ids[3:6]) == [0, 2, 5]
    info, x = oracle.sample_row_ex(z, np.zeros_like(z), 0.0, 1.0, 0,
                                   mask=np.array([1, 0, 1, 0, 0, 1], np.uint8))
    assert info.id == 2 and x.chosen_prob == 1.0


def test_masked_draws_follow_renormalised_softmax():
    """Chi-square over 40000 draws with a mask and top-k 4: ids follow the
    softmax of the scaled logits restricted to the allowed top-4."""
    rng = np.random.default_rng(94)
    V, N = 10, 40000
    z = np.array([2.5, 2.0, 1.8, 1.0, 0.7, 0.5, 0.0, -0.4, -1.0, -2.0], np.float32)
    mask = np.array([0, 1, 1, 0, 1, 1, 1, 1, 0, 1], np.uint8)
    T = np.float32(0.9)
    allowed = np.nonzero(mask)[0]
    top = allowed[np.argsort(-(z[allowed] / T), kind="stable")[:4]]
    probs = _softmax64((z[top] / T).astype(np.float64))
    counts = np.zeros(V, np.int64)
    for _ in range(N):
        g = rng.gumbel(size=V).astype(np.float32)
        info, _ = oracle.sample_row_ex(z, g, T, 1.0, 4, mask=mask)
        counts[info.id] += 1
    assert counts.sum() == counts[top].sum()
    exp_ = probs * N
    chi2 = float(np.sum((counts[top] - exp_) ** 2 / exp_))
    assert chi2 < 16.3, (chi2, counts[top], exp_)   # 99.9% quantile, 3 dof


# ------------------------------------------ varlen multi-query attention --

def _varlen_case(rng, lens_new, lens_cached, H, Hkv, D, bs):
    """Whole sequences (cached + new tokens) in a fragmented paged cache;
    returns the dense per-sequence tensors and the varlen arguments."""
    B = len(lens_new)
    total = [c + q for c, q in zip(lens_cached, lens_new)]
    need = [(n + bs - 1) // bs for n in total]
    nb = sum(need) + 2
    perm = rng.permutation(nb).astype(np.int32)
    W = max(need)
    tables = np.full((B, W), -1, np.int32)
    kc = _bf16(rng, (nb, bs, Hkv, D))
    vc = _bf16(rng, (nb, bs, Hkv, D))
    seqs = []
    pos = 0
    for b in range(B):
        tables[b, :need[b]] = perm[pos:pos + need[b]]
        pos += need[b]
        n = total[b]
        qs, ks, vs = _bf16(rng, (n, H, D)), _bf16(rng, (n, Hkv, D)), _bf16(rng, (n, Hkv, D))
        for j in range(n):
            s = oracle.slot_for_position(tables[b], j, bs)
            kc.reshape(-1, Hkv, D)[s] = ks[j]
            vc.reshape(-1, Hkv, D)[s] = vs[j]
        seqs.append((qs, ks, vs))
    cu_q = np.concatenate([[0], np.cumsum(lens_new)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(total)]).astype(np.int32)
    q = np.concatenate([seqs[b][0][lens_cached[b]:] for b in range(B)], axis=0)
    return seqs, q, kc, vc, tables, cu_q, cu_k


def test_varlen_rows_equal_dense_causal_attention():
    """Each new token of a chunk (cached prefix + new tokens, several
    sequences of different lengths) reproduces its row of full causal
    attention over the whole sequence, computed as one masked matrix."""
    rng = np.random.default_rng(140)
    H, Hkv, D, bs = 6, 2, 8, 4
    lens_new = [5, 1, 9, 3]
    lens_cached = [0, 6, 13, 2]
    seqs, q, kc, vc, tables, cu_q, cu_k = _varlen_case(rng, lens_new, lens_cached, H, Hkv, D, bs)
    got = oracle.varlen_attention(q, kc, vc, tables, cu_q, cu_k)
    for b, (qs, ks, vs) in enumerate(seqs):
        ref = _causal_last_rows(f32_from_bf16_bits(qs).astype(np.float64),
                                f32_from_bf16_bits(ks).astype(np.float64),
                                f32_from_bf16_bits(vs).astype(np.float64), 1.0 / math.sqrt(D))
        np.testing.assert_allclose(got[cu_q[b]:cu_q[b + 1]], ref[lens_cached[b]:], rtol=0,
                                   atol=1e-12)


def test_varlen_chunked_prefill_equals_one_chunk():
    """A prefill cut into chunks (each later chunk seeing the earlier ones
    as its cached prefix) gives the same rows as one chunk."""
    rng = np.random.default_rng(141)
    H, Hkv, D, bs = 4, 4, 8, 8
    n = 37
    seqs, q, kc, vc, tables, cu_q, cu_k = _varlen_case(rng, [n], [0], H, Hkv, D, bs)
    whole = oracle.varlen_attention(q, kc, vc, tables, cu_q, cu_k)
    parts = []
    start = 0
    for step in (10, 1, 20, 6):
        cq = np.array([0, step], np.int32)
        ck = np.array([0, start + step], np.int32)
        parts.append(oracle.varlen_attention(q[start:start + step], kc, vc, tables, cq, ck))
        start += step
    np.testing.assert_array_equal(np.concatenate(parts), whole)


def test_varlen_slot_mapping_covers_the_new_positions():
    rng = np.random.default_rng(142)
    bs = 4
    lens_new, lens_cached = [3, 1, 6], [5, 0, 8]
    seqs, q, kc, vc, tables, cu_q, cu_k = _varlen_case(rng, lens_new, lens_cached, 2, 1, 8, bs)
    slots = oracle.varlen_slot_mapping(tables, cu_q, cu_k, bs)
    for b in range(3):
        for j in range(lens_new[b]):
            pos = lens_cached[b] + j
            assert slots[cu_q[b] + j] == tables[b, pos // bs] * bs + pos % bs
    # one new token per sequence: the decode slot mapping
    cq = np.arange(4, dtype=np.int32)
    ck = np.concatenate([[0], np.cumsum([8, 1, 14])]).astype(np.int32)
    np.testing.assert_array_equal(oracle.varlen_slot_mapping(tables, cq, ck, bs),
                                  oracle.slot_mapping(tables, np.array([8, 1, 14], np.int32), bs))
