"""Pins for the oracle's method steps.

Each test compares the oracle with something it does not share code with:
the Vortex post's Fig. 1 worked example (tests/golden), brute-force subset
enumeration, exact rationals (fractions.Fraction), 50-digit decimal softmax
computed without the max shift, closed forms (one token, equal logits),
invariants (shift, permutation of physical pages, convexity), and the
log-sum-exp merge of attention over disjoint token sets.
"""

import itertools
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

from oracle.method import (
    BatchView, attention_over_tokens, block_bounds, block_scores, block_summaries,
    bound_scores, coarse_to_fine_select,
    decode_step,
    dense_attention, forced_blocks, indexer_block_scores, indexer_token_scores, lse_merge,
    mla_attention, select_blocks, select_tokens, sparse_attention, tokens_of_blocks,
)
from oracle.numerics import (
    bf16_to_f64, f64_to_bf16_bits, fp8e4m3fn_to_f64, fraction_to_bf16_bits, fraction_to_f32,
)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rest = line.split(":", 1)
            vals[key.strip()] = rest.split()
    return vals


def _rand_bf16(rng, shape, scale=1.0):
    return f64_to_bf16_bits(rng.standard_normal(shape) * scale)


# ---------------------------------------------------------------- selection

def test_vortex_fig1_example():
    g = _read_golden("vortex_fig1_block_scores.txt")
    scores = np.array([float(x) for x in g["scores"]])
    k = int(g["k"][0])
    kept = [int(x) for x in g["kept"]]
    assert select_blocks(scores, nb=8, n_complete=8, k=k, n_sink=0, n_recent=0) == kept
    # unchanged after rounding the scores to bf16 (values stay distinct)
    s16 = bf16_to_f64(f64_to_bf16_bits(scores))
    assert len(set(s16.tolist())) == 8
    assert select_blocks(s16, nb=8, n_complete=8, k=k, n_sink=0, n_recent=0) == kept


def _brute_topk(scores, cands, k):
    """The unique k-subset T of cands with every member ahead of every
    non-member under (score desc, index asc), found by enumeration."""
    found = []
    for T in itertools.combinations(cands, min(k, len(cands))):
        rest = [b for b in cands if b not in T]
        if all(scores[a] > scores[b] or (scores[a] == scores[b] and a < b)
               for a in T for b in rest):
            found.append(set(T))
    assert len(found) == 1
    return found[0]


def test_selection_vs_subset_enumeration_with_ties():
    rng = np.random.default_rng(10)
    for trial in range(300):
        nb = int(rng.integers(1, 11))
        partial = bool(rng.integers(0, 2)) and nb > 0
        n_complete = nb - 1 if partial else nb
        scores = rng.integers(-3, 4, n_complete).astype(np.float64)   # many ties
        k = int(rng.integers(0, 6))
        n_sink = int(rng.integers(0, 3))
        n_recent = int(rng.integers(0, 3))
        got = select_blocks(scores, nb, n_complete, k, n_sink, n_recent)
        forced = set(range(min(n_sink, nb))) | set(range(max(0, nb - n_recent), nb))
        if partial:
            forced.add(nb - 1)
        cands = [b for b in range(n_complete) if b not in forced]
        want = forced | _brute_topk(scores, cands, k)
        assert got == sorted(want), (trial, scores, k, n_sink, n_recent)
        assert got == sorted(set(got))


def test_selection_all_blocks_when_budget_covers_everything():
    scores = np.array([5.0, 1.0, 3.0, 2.0])
    assert select_blocks(scores, 5, 4, k=10, n_sink=1, n_recent=2) == [0, 1, 2, 3, 4]
    assert forced_blocks(5, 4, 1, 0) == [0, 4]             # partial last block forced
    assert forced_blocks(3, 3, 2, 2) == [0, 1, 2]          # overlap de-duplicated
    assert forced_blocks(0, 0, 1, 2) == []


def test_duplicated_scores_pick_lowest_index():
    scores = np.full(10, 7.0)
    assert select_blocks(scores, 10, 10, k=3, n_sink=0, n_recent=0) == [0, 1, 2]
    assert select_blocks(scores, 10, 10, k=3, n_sink=1, n_recent=1) == [0, 1, 2, 3, 9]


def test_token_selection_vs_enumeration():
    rng = np.random.default_rng(11)
    for _ in range(100):
        n = int(rng.integers(1, 10))
        s = rng.integers(-2, 3, n).astype(np.float64)
        k = int(rng.integers(0, 5))
        assert select_tokens(s, k) == sorted(_brute_topk(s, list(range(n)), k))


# ---------------------------------------------------------------- summaries

def test_summaries_vs_exact_rational_mean():
    rng = np.random.default_rng(12)
    pool = _rand_bf16(rng, (5, 3, 16, 8))
    got = block_summaries(pool, [0, 2, 4])
    vals = bf16_to_f64(pool)
    for i, p in enumerate([0, 2, 4]):
        for h in range(3):
            for d in range(8):
                mean = sum(Fraction(float(v)) for v in vals[p, h, :, d]) / 16
                assert got[i, h, d] == fraction_to_bf16_bits(mean)
    got32 = block_summaries(pool, [1], out_dtype="fp32")
    mean = sum(Fraction(float(v)) for v in vals[1, 0, :, 0]) / 16
    assert got32[0, 0, 0] == fraction_to_f32(mean)


def test_summaries_constant_tile_and_inexact_fallback():
    pool = np.full((2, 1, 16, 4), 0x4040, dtype=np.uint16)     # 3.0 everywhere
    assert np.all(block_summaries(pool, [0, 1]) == 0x4040)
    # a column whose float64 sum would lose bits: 2^100, tiny values, -2^100
    col = np.zeros(16)
    col[0], col[1], col[2] = 2.0 ** 100, 2.0 ** -100, -(2.0 ** 100)
    col[3] = 3.0 * 2.0 ** -100
    pool = np.zeros((1, 1, 16, 1), dtype=np.uint16)
    pool[0, 0, :, 0] = f64_to_bf16_bits(col)
    got = block_summaries(pool, [0])
    exact = sum(Fraction(float(v)) for v in bf16_to_f64(pool[0, 0, :, 0])) / 16
    assert got[0, 0, 0] == fraction_to_bf16_bits(exact)
    assert bf16_to_f64(got[0, 0, 0]) == 2.0 ** -100 / 4     # (1 + 3) * 2^-100 / 16


def test_fp8_indexer_summaries_vs_rationals():
    rng = np.random.default_rng(13)
    keys = rng.integers(0, 256, (3, 64, 4)).astype(np.uint8)
    keys[(keys & 0x7F) == 0x7F] = 0x10                         # no NaN codes
    scales = (rng.random((3, 64)) * 0.01 + 1e-3).astype(np.float32)
    got = block_summaries(keys, [0, 2], key_format="fp8_e4m3fn", key_scales=scales)
    for i, p in enumerate([0, 2]):
        for d in range(4):
            mean = sum(Fraction(float(scales[p, s])) * Fraction(float(fp8e4m3fn_to_f64(keys[p, s, d])))
                       for s in range(64)) / 64
            assert got[i, d] == fraction_to_bf16_bits(mean)


# ---------------------------------------------------------------- scores

def _tiny_batch(rng, B=2, Hq=4, Hkv=2, D=8, P=4, lens=(13, 8), num_pages=None):
    nbs = [(L + P - 1) // P for L in lens]
    used = sum(nbs)
    num_pages = num_pages or used + 3
    phys = rng.permutation(num_pages)[:used]
    indptr = np.concatenate([[0], np.cumsum(nbs)])
    return BatchView(indptr, phys, np.array(lens), P), num_pages


def test_block_scores_vs_exact_rationals():
    rng = np.random.default_rng(14)
    batch, npg = _tiny_batch(rng)
    q = _rand_bf16(rng, (2, 4, 8))
    summ = _rand_bf16(rng, (npg, 2, 8))
    for r in range(2):
        for g in range(2):
            for agg in ("max", "mean"):
                s = block_scores(q, summ, batch, r, g, num_kv_heads=2, agg=agg)
                nc = batch.num_complete(r)
                assert s.shape == (nc,)
                for j in range(nc):
                    p = batch.pages(r)[j]
                    dots = [sum(Fraction(float(a)) * Fraction(float(b)) for a, b in
                                zip(bf16_to_f64(q[r, h]), bf16_to_f64(summ[p, g])))
                            for h in (2 * g, 2 * g + 1)]
                    want = max(dots) if agg == "max" else sum(dots) / 2
                    assert abs(Fraction(float(s[j])) - want) <= abs(want) * Fraction(1, 10 ** 14) + Fraction(1, 10 ** 300)


# ------------------------------------------------------------ Quest bounds

def test_quest_worked_example():
    # one head, one 2-token block: k1 = (3, 1), k2 = (-1, 4) -> max (3, 4),
    # min (-1, 1); q = (1, -2): max(1*3, 1*-1) + max(-2*4, -2*1) = 3 - 2 = 1,
    # while the tokens' own dot products are 1 and -9
    keys = f64_to_bf16_bits(np.array([[[[3.0, 1.0], [-1.0, 4.0]]]]))       # [1][1][2][2]
    b = block_bounds(keys, [0])
    assert b.shape == (1, 1, 2, 2)
    assert bf16_to_f64(b[0, 0, 0]).tolist() == [3.0, 4.0]
    assert bf16_to_f64(b[0, 0, 1]).tolist() == [-1.0, 1.0]
    q = f64_to_bf16_bits(np.array([[[1.0, -2.0]]]))
    batch = BatchView([0, 1], [0], [2], 2)
    s = bound_scores(q, b, batch, 0, 0, num_kv_heads=1)
    assert s.tolist() == [1.0]


def test_quest_score_is_the_max_over_the_box_corners():
    # the largest q . x over the box [min, max] sits at a corner: enumerate
    # all 2^D corners with exact rationals
    rng = np.random.default_rng(31)
    D, P = 6, 4
    keys = _rand_bf16(rng, (3, 1, P, D))
    b = block_bounds(keys, [0, 1, 2])
    q = _rand_bf16(rng, (1, 1, D))
    batch = BatchView([0, 3], [0, 1, 2], [3 * P], P)
    s = bound_scores(q, b, batch, 0, 0, num_kv_heads=1)
    qf = [Fraction(float(x)) for x in bf16_to_f64(q[0, 0])]
    for j in range(3):
        hi = [Fraction(float(x)) for x in bf16_to_f64(b[j, 0, 0])]
        lo = [Fraction(float(x)) for x in bf16_to_f64(b[j, 0, 1])]
        best = max(sum(qf[d] * (hi[d] if (c >> d) & 1 else lo[d]) for d in range(D))
                   for c in range(2 ** D))
        assert Fraction(float(s[j])) == best          # few exact products: no rounding


def test_quest_bounds_and_scores_bound_every_token():
    rng = np.random.default_rng(32)
    batch, npg = _tiny_batch(rng)
    keys = _rand_bf16(rng, (npg, 2, 4, 8))
    q = _rand_bf16(rng, (2, 4, 8))
    b = block_bounds(keys, range(npg))
    for p in range(npg):
        for h in range(2):
            for d in range(8):
                col = [Fraction(float(x)) for x in bf16_to_f64(keys[p, h, :, d])]
                assert Fraction(float(bf16_to_f64(b[p, h, 0, d]))) == max(col)
                assert Fraction(float(bf16_to_f64(b[p, h, 1, d]))) == min(col)
    for r in range(2):
        for g in range(2):
            # head 2g + i alone: both of the group's slots hold it
            per_head = []
            for i in range(2):
                qq = q.copy()
                qq[:, 2 * g] = qq[:, 2 * g + 1] = q[:, 2 * g + i]
                per_head.append(bound_scores(qq, b, batch, r, g, num_kv_heads=2))
            s = bound_scores(q, b, batch, r, g, num_kv_heads=2, agg="max")
            assert np.array_equal(s, np.maximum(per_head[0], per_head[1]))
            for j in range(batch.num_complete(r)):
                p = batch.pages(r)[j]
                for i in range(2):
                    qh = [Fraction(float(x)) for x in bf16_to_f64(q[r, 2 * g + i])]
                    for t in range(4):
                        kt = [Fraction(float(x)) for x in bf16_to_f64(keys[p, g, t])]
                        dot = sum(a * c for a, c in zip(qh, kt))
                        assert dot <= Fraction(float(per_head[i][j])) * (1 + Fraction(1, 10 ** 12)) + Fraction(1, 10 ** 300)


def test_quest_block_of_equal_tokens_scores_its_dot_product():
    rng = np.random.default_rng(33)
    tok = _rand_bf16(rng, (8,))
    keys = np.broadcast_to(tok, (1, 1, 4, 8)).copy()
    b = block_bounds(keys, [0])
    assert np.array_equal(b[0, 0, 0], tok) and np.array_equal(b[0, 0, 1], tok)
    q = _rand_bf16(rng, (1, 1, 8))
    batch = BatchView([0, 1], [0], [4], 4)
    s = bound_scores(q, b, batch, 0, 0, num_kv_heads=1)
    want = sum(Fraction(float(a)) * Fraction(float(c))
               for a, c in zip(bf16_to_f64(q[0, 0]), bf16_to_f64(tok)))
    assert abs(Fraction(float(s[0])) - want) <= abs(want) * Fraction(1, 10 ** 14)


def test_quest_step_finds_the_block_of_a_planted_key():
    """A key aligned with a query head, planted in one block of each request
    among small keys: the Quest step (bounds, top-1 + 1 recent) keeps that
    block, and its attention is the attention over the kept blocks."""
    rng = np.random.default_rng(34)
    batch, npg = _tiny_batch(rng, lens=(24, 20))
    keys = _rand_bf16(rng, (npg, 2, 4, 8), scale=0.05)
    vals = _rand_bf16(rng, (npg, 2, 4, 8))
    q = _rand_bf16(rng, (2, 4, 8))
    planted = {0: 2, 1: 1}                      # request -> block holding the key
    for r, j in planted.items():
        p = batch.pages(r)[j]
        keys[p, 1, 3] = f64_to_bf16_bits(4 * bf16_to_f64(q[r, 3]))   # kv head 1, head 3
    res = decode_step(q, keys, vals, batch, num_kv_heads=2, topk=1, n_sink=0, n_recent=1,
                      sm_scale=0.25, score_mode="bounds", out_dtype="fp64")
    for r, j in planted.items():
        nb = batch.num_blocks(r)
        got = res["pairs"][(r, 1)]
        assert got["selected"] == sorted({j, nb - 1})
        o, lse = sparse_attention(q, keys, vals, batch, r, 1, got["selected"], num_kv_heads=2,
                                  sm_scale=0.25, out_dtype="fp64")
        assert np.array_equal(o, got["out"]) and np.array_equal(lse, got["lse"])
    assert res["summaries"].shape == (npg, 2, 2, 8)


def test_max_and_mean_agree_for_one_head_per_group():
    rng = np.random.default_rng(15)
    batch, npg = _tiny_batch(rng, Hq=2, Hkv=2)
    q = _rand_bf16(rng, (2, 2, 8))
    summ = _rand_bf16(rng, (npg, 2, 8))
    a = block_scores(q, summ, batch, 0, 1, num_kv_heads=2, agg="max")
    b = block_scores(q, summ, batch, 0, 1, num_kv_heads=2, agg="mean")
    assert np.array_equal(a, b)


def test_indexer_scores_vs_rationals_and_homogeneity():
    rng = np.random.default_rng(16)
    batch, npg = _tiny_batch(rng, lens=(9, 4), P=4)
    keys = rng.integers(0, 256, (npg, 4, 6)).astype(np.uint8)
    keys[(keys & 0x7F) == 0x7F] = 0x31
    scales = (rng.random((npg, 4)) + 0.5).astype(np.float32)
    q = _rand_bf16(rng, (2, 3, 6))
    w = rng.standard_normal((2, 3)).astype(np.float32)
    s = indexer_token_scores(q, w, keys, scales, batch, 0)
    for t in range(9):
        p, sl = batch.pages(0)[t // 4], t % 4
        k = [Fraction(float(scales[p, sl])) * Fraction(float(v)) for v in fp8e4m3fn_to_f64(keys[p, sl])]
        want = Fraction(0)
        for h in range(3):
            dot = sum(Fraction(float(a)) * b for a, b in zip(bf16_to_f64(q[0, h]), k))
            want += Fraction(float(w[0, h])) * max(dot, Fraction(0))
        assert abs(Fraction(float(s[t])) - want) <= abs(want) * Fraction(1, 10 ** 13) + Fraction(1, 10 ** 300)
    # ReLU is positively homogeneous: doubling a token's scale doubles its score
    scales2 = scales.copy()
    p0 = batch.pages(0)[0]
    scales2[p0, 1] *= 2
    s2 = indexer_token_scores(q, w, keys, scales2, batch, 0)
    assert s2[1] == 2 * s[1]
    assert np.array_equal(np.delete(s2, 1), np.delete(s, 1))
    # block form on summaries: Eq. 6 applied to the block-mean keys, written
    # over rationals by the brute force below (its own decoder, its own walk
    # of the page table)
    summ = _rand_bf16(rng, (npg, 6))
    for r in range(2):
        sb = indexer_block_scores(q, w, summ, batch, r)
        want = _fraction_indexer_block_scores(q, w, summ, batch, r)
        assert sb.shape == (len(want),) == (int(batch.seq_lens[r]) // 4,)
        for got, ref in zip(sb, want):
            assert abs(Fraction(float(got)) - ref) <= abs(ref) * Fraction(1, 10 ** 13) + Fraction(1, 10 ** 300)


def _bf16_bits_to_fraction(bits):
    """Exact value of a bf16 bit pattern (finite), from the IEEE fields."""
    bits = int(bits) & 0xFFFF
    sign = -1 if bits >> 15 else 1
    exp, man = (bits >> 7) & 0xFF, bits & 0x7F
    assert exp != 0xFF
    if exp == 0:
        return sign * Fraction(man, 1 << 7) * Fraction(1, 1 << 126)
    v = Fraction((1 << 7) + man, 1 << 7)
    e = exp - 127
    return sign * (v * (1 << e) if e >= 0 else v / (1 << -e))


def _fraction_indexer_block_scores(q_bits, w, summ_bits, batch, r):
    """s_j = sum_h w_h * max(0, q_h . kbar_j) over the complete blocks j of
    request r (LeanSparse §5, Eq. 6 on block-mean keys), in rationals, with
    block j's summary at row page_indices[page_indptr[r] + j]."""
    P = batch.page_size
    nc = int(batch.seq_lens[r]) // P
    base = int(batch.page_indptr[r])
    out = []
    for j in range(nc):
        page = int(batch.page_indices[base + j])
        kbar = [_bf16_bits_to_fraction(b) for b in np.asarray(summ_bits)[page]]
        total = Fraction(0)
        for h in range(q_bits.shape[1]):
            qh = [_bf16_bits_to_fraction(b) for b in q_bits[r, h]]
            dot = sum((a * b for a, b in zip(qh, kbar)), Fraction(0))
            total += Fraction(float(w[r, h])) * max(dot, Fraction(0))
        out.append(total)
    return out


def test_indexer_block_scores_brute_force_catches_plausible_mistakes():
    """The rational brute force separates the oracle's block score from the
    nearby wrong readings: logical instead of physical page, ReLU after the
    head sum, unweighted heads."""
    rng = np.random.default_rng(161)
    batch, npg = _tiny_batch(rng, lens=(28,), P=4)
    q = _rand_bf16(rng, (1, 3, 6))
    w = rng.standard_normal((1, 3)).astype(np.float32)
    summ = _rand_bf16(rng, (npg, 6))
    ref = [float(x) for x in _fraction_indexer_block_scores(q, w, summ, batch, 0)]
    got = indexer_block_scores(q, w, summ, batch, 0)
    assert np.allclose(got, ref, rtol=1e-13, atol=0)
    S = bf16_to_f64(summ)
    qq = bf16_to_f64(q[0])
    ww = w[0].astype(np.float64)
    logical = np.maximum(S[: len(ref)] @ qq.T, 0.0) @ ww
    late_relu = np.maximum((S[batch.pages(0)[: len(ref)]] @ qq.T) @ ww, 0.0)
    unweighted = np.maximum(S[batch.pages(0)[: len(ref)]] @ qq.T, 0.0).sum(axis=1)
    for wrong in (logical, late_relu, unweighted):
        assert not np.allclose(wrong, ref, rtol=1e-9, atol=0)


# ---------------------------------------------------------------- attention

getcontext().prec = 50


def _decimal_attention(q, K, V, scale):
    """softmax attention without the max shift, in 50-digit decimal."""
    z = [Decimal(float(scale)) * sum(Decimal(float(a)) * Decimal(float(b)) for a, b in zip(q, k))
         for k in K]
    e = [x.exp() for x in z]
    Z = sum(e)
    o = [sum(e[t] * Decimal(float(V[t][d])) for t in range(len(V))) / Z for d in range(len(V[0]))]
    return np.array([float(x) for x in o]), float(Z.ln())


def test_attention_vs_decimal_brute_force():
    rng = np.random.default_rng(17)
    for T in (1, 2, 7, 33):
        q = rng.standard_normal(8)
        K = rng.standard_normal((T, 8)) * 2
        V = rng.standard_normal((T, 5))
        o, lse = attention_over_tokens(q, K, V, 0.35)
        o2, lse2 = _decimal_attention(q, K, V, 0.35)
        np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-13)
        assert abs(lse - lse2) < 1e-12


def test_attention_closed_forms_and_invariants():
    rng = np.random.default_rng(18)
    V = rng.standard_normal((6, 4))
    K = rng.standard_normal((6, 4))
    # one token -> exactly its value
    o, _ = attention_over_tokens(rng.standard_normal(4), K[:1], V[:1], 0.5)
    assert np.array_equal(o, V[0])
    # equal logits -> mean of values
    o, lse = attention_over_tokens(np.zeros(4), K, V, 0.5)
    np.testing.assert_allclose(o, V.mean(axis=0), rtol=0, atol=1e-15)
    assert abs(lse - math.log(6)) < 1e-15
    # weights sum to one: all-ones values give ones
    o, _ = attention_over_tokens(rng.standard_normal(4), K, np.ones((6, 3)), 0.5)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-15)
    # convex combination: inside [min V, max V]
    o, _ = attention_over_tokens(rng.standard_normal(4) * 5, K, V, 1.0)
    assert np.all(o >= V.min(axis=0) - 1e-15) and np.all(o <= V.max(axis=0) + 1e-15)
    # a constant shift of every logit leaves o unchanged and moves lse
    q = rng.standard_normal(4)
    o1, l1 = attention_over_tokens(q, K, V, 0.5)
    o2, l2 = attention_over_tokens(np.append(q, 3.0), np.hstack([K, np.ones((6, 1))]), V, 0.5)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-14)
    assert abs((l2 - l1) - 1.5) < 1e-13
    # empty set
    o, lse = attention_over_tokens(q, K[:0], V[:0], 0.5)
    assert np.all(o == 0) and lse == -np.inf


def test_lse_merge_equals_attention_over_union():
    rng = np.random.default_rng(19)
    q = rng.standard_normal(8)
    K = rng.standard_normal((40, 8)) * 1.5
    V = rng.standard_normal((40, 6))
    whole = attention_over_tokens(q, K, V, 0.4)
    cuts = [0, 3, 17, 18, 40]
    parts = [attention_over_tokens(q, K[a:b], V[a:b], 0.4) for a, b in zip(cuts, cuts[1:])]
    merged = lse_merge(parts)
    np.testing.assert_allclose(merged[0], whole[0], rtol=1e-13, atol=1e-14)
    assert abs(merged[1] - whole[1]) < 1e-13
    # an empty part changes nothing
    merged2 = lse_merge(parts + [attention_over_tokens(q, K[:0], V[:0], 0.4)])
    np.testing.assert_allclose(merged2[0], whole[0], rtol=1e-13, atol=1e-14)


def _paged_tiny(rng, lens=(21, 16, 5), Hq=4, Hkv=2, D=8, P=4, extra_pages=3):
    nbs = [(L + P - 1) // P for L in lens]
    used = sum(nbs)
    npg = used + extra_pages
    phys = rng.permutation(npg)[:used]
    indptr = np.concatenate([[0], np.cumsum(nbs)])
    batch = BatchView(indptr, phys, np.array(lens), P)
    q = _rand_bf16(rng, (len(lens), Hq, D))
    k = _rand_bf16(rng, (npg, Hkv, P, D))
    v = _rand_bf16(rng, (npg, Hkv, P, D))
    return batch, q, k, v


def test_k_all_equals_dense_decimal_attention():
    rng = np.random.default_rng(20)
    batch, q, k, v = _paged_tiny(rng)
    for r in range(batch.batch):
        L = int(batch.seq_lens[r])
        for g in range(2):
            out, lse = dense_attention(q, k, v, batch, r, g, num_kv_heads=2, sm_scale=0.3,
                                       out_dtype="fp64")
            # contiguous view of the request's tokens, built independently
            Kc = np.stack([bf16_to_f64(k[batch.page_indices[batch.page_indptr[r] + t // 4], g, t % 4])
                           for t in range(L)])
            Vc = np.stack([bf16_to_f64(v[batch.page_indices[batch.page_indptr[r] + t // 4], g, t % 4])
                           for t in range(L)])
            for i, h in enumerate((2 * g, 2 * g + 1)):
                o2, l2 = _decimal_attention(bf16_to_f64(q[r, h]), Kc, Vc, 0.3)
                np.testing.assert_allclose(out[i], o2, rtol=1e-12, atol=1e-13)
                assert abs(lse[i] - l2) < 1e-12


def test_page_permutation_invariance_and_poisoned_unused_pages():
    rng = np.random.default_rng(21)
    batch, q, k, v = _paged_tiny(rng)
    res1 = decode_step(q, k, v, batch, num_kv_heads=2, topk=2, n_sink=1, n_recent=1,
                       sm_scale=0.3, out_dtype="bf16")
    # move every page to a new physical slot and poison the unused ones
    npg = k.shape[0]
    perm = rng.permutation(npg + 4)
    k2 = np.full((npg + 4,) + k.shape[1:], 0x7FC0, dtype=np.uint16)
    v2 = np.full_like(k2, 0x7FC0)
    k2[perm[:npg]] = k
    v2[perm[:npg]] = v
    batch2 = BatchView(batch.page_indptr, perm[batch.page_indices], batch.seq_lens, 4)
    res2 = decode_step(q, k2, v2, batch2, num_kv_heads=2, topk=2, n_sink=1, n_recent=1,
                       sm_scale=0.3, out_dtype="bf16")
    for key, a in res1["pairs"].items():
        b = res2["pairs"][key]
        assert a["selected"] == b["selected"]
        assert np.array_equal(a["out"], b["out"])
        assert np.array_equal(a["scores"], b["scores"])


def test_decode_step_k_all_matches_dense():
    rng = np.random.default_rng(22)
    batch, q, k, v = _paged_tiny(rng)
    res = decode_step(q, k, v, batch, num_kv_heads=2, topk=100, n_sink=1, n_recent=2,
                      sm_scale=0.3, out_dtype="fp32")
    for (r, g), item in res["pairs"].items():
        assert item["selected"] == list(range(batch.num_blocks(r)))
        out, lse = dense_attention(q, k, v, batch, r, g, num_kv_heads=2, sm_scale=0.3,
                                   out_dtype="fp32")
        assert np.array_equal(item["out"], out)


def test_sparse_attention_is_lse_merge_of_its_blocks():
    rng = np.random.default_rng(23)
    batch, q, k, v = _paged_tiny(rng)
    blocks = [0, 2, 5]
    out, lse = sparse_attention(q, k, v, batch, 0, 1, blocks, num_kv_heads=2, sm_scale=0.3,
                                out_dtype="fp64")
    parts = [sparse_attention(q, k, v, batch, 0, 1, [b], num_kv_heads=2, sm_scale=0.3,
                              out_dtype="fp64") for b in blocks]
    for i in range(2):
        o, l = lse_merge([(p[0][i], p[1][i]) for p in parts])
        np.testing.assert_allclose(out[i], o, rtol=1e-13, atol=1e-14)
        assert abs(lse[i] - l) < 1e-13
    assert list(tokens_of_blocks([5], 4, 21)) == [20]


def test_mla_attention_vs_decimal():
    rng = np.random.default_rng(24)
    lens = (10,)
    batch = BatchView([0, 3], [2, 0, 1], np.array(lens), 4)
    lat = _rand_bf16(rng, (3, 4, 6))          # Dk = 6, v_dim = 4
    q = _rand_bf16(rng, (1, 3, 6))
    toks = [0, 4, 5, 9]
    out, lse = mla_attention(q, lat, batch, 0, toks, v_dim=4, sm_scale=0.5, out_dtype="fp64")
    C = np.stack([bf16_to_f64(lat[batch.page_indices[t // 4], t % 4]) for t in toks])
    for h in range(3):
        o2, l2 = _decimal_attention(bf16_to_f64(q[0, h]), C, C[:, :4], 0.5)
        np.testing.assert_allclose(out[h], o2, rtol=1e-12, atol=1e-13)
        assert abs(lse[h] - l2) < 1e-12


def test_keep_ratio_budget_closed_forms():
    from oracle.method import topk_from_keep_ratio
    # ratio 1 keeps every block: k = every candidate
    assert topk_from_keep_ratio(100, 100, 1.0, 1, 2) == 97
    assert topk_from_keep_ratio(100, 99, 1.0, 1, 2) == 97      # partial last is recent
    # 1/16 of 2048 blocks = 128 kept in all, 3 of them forced
    assert topk_from_keep_ratio(2048, 2048, 1 / 16, 1, 2) == 125
    # a budget below the forced count keeps only the forced blocks
    assert topk_from_keep_ratio(10, 10, 1 / 64, 1, 2) == 0
    # ceil: 1/64 of 130 = 2.03 -> 3 kept in all, 3 forced -> k = 0; of 200 -> 4 -> k = 1
    assert topk_from_keep_ratio(130, 130, 1 / 64, 1, 2) == 0
    assert topk_from_keep_ratio(200, 200, 1 / 64, 1, 2) == 1


# ------------------------------------------------------------ coarse-to-fine

def _indexer_problem(rng, lens, P, H=3, D=6):
    batch, npg = _tiny_batch(rng, lens=lens, P=P)
    keys = rng.integers(0, 256, (npg, P, D)).astype(np.uint8)
    keys[(keys & 0x7F) == 0x7F] = 0x31          # no NaN encodings
    scales = (rng.random((npg, P)) + 0.5).astype(np.float32)
    q = _rand_bf16(rng, (len(lens), H, D))
    w = rng.standard_normal((len(lens), H)).astype(np.float32)
    summ = block_summaries(keys, range(npg), key_format="fp8_e4m3fn", key_scales=scales)
    return batch, keys, scales, q, w, summ


def test_coarse_to_fine_with_every_block_kept_is_exact_token_topk():
    rng = np.random.default_rng(31)
    batch, keys, scales, q, w, summ = _indexer_problem(rng, lens=(37, 16), P=4)
    for r in range(2):
        L = int(batch.seq_lens[r])
        res = coarse_to_fine_select(q, w, keys, scales, summ, batch, r,
                                    topk_blocks=batch.num_blocks(r), n_recent_blocks=1,
                                    topk_tokens=5)
        assert res["blocks"] == list(range(batch.num_blocks(r)))
        s = indexer_token_scores(q, w, keys, scales, batch, r)
        # pairwise dominance characterises the top-k set: every kept token
        # beats every dropped token under (score desc, token asc)
        kept = set(res["tokens"])
        assert len(kept) == min(5, L)
        for a in kept:
            for b in set(range(L)) - kept:
                assert s[a] > s[b] or (s[a] == s[b] and a < b)


def test_coarse_to_fine_never_leaves_the_kept_blocks():
    rng = np.random.default_rng(32)
    batch, keys, scales, q, w, summ = _indexer_problem(rng, lens=(64,), P=4)
    res = coarse_to_fine_select(q, w, keys, scales, summ, batch, 0, topk_blocks=3,
                                n_recent_blocks=1, topk_tokens=6)
    nb = batch.num_blocks(0)
    assert len(res["blocks"]) == 4 and nb - 1 in res["blocks"]
    # the coarse pass ranks blocks by the block-mean score (rational brute force)
    sb = _fraction_indexer_block_scores(q, w, summ, batch, 0)
    cands = [j for j in range(nb) if j != nb - 1]
    top = sorted(cands, key=lambda j: (-sb[j], j))[:3]
    assert sorted(top + [nb - 1]) == res["blocks"]
    allowed = set(tokens_of_blocks(res["blocks"], 4, 64).tolist())
    assert set(res["tokens"]) <= allowed and len(res["tokens"]) == 6
    # among the kept blocks' tokens the choice is the exact top-6
    s = indexer_token_scores(q, w, keys, scales, batch, 0)
    for a in res["tokens"]:
        for b in allowed - set(res["tokens"]):
            assert s[a] > s[b] or (s[a] == s[b] and a < b)


# ------------------------------------------------------- approximate top-k

def test_remap_bucket_hand_worked():
    from oracle.method import remap_bucket
    # mn 0, mx 4: scale = 4096 / 4 = 1024, t = 1024 s; the largest score lands
    # on t = 4096 and is clamped into the top bucket 4095
    s = np.array([0.0, 4.0, 2.0, 2.0005, 1.0])
    assert remap_bucket(s).tolist() == [0, 4095, 2048, 2048, 1024]
    # an offset range: mn -3, span 4, the same scale
    assert remap_bucket(np.array([-3.0, -1.0, 1.0, -2.5])).tolist() == [0, 2048, 4095, 512]
    # span 4096: scale 1, every integer its own bucket, the top two clamped
    s = np.arange(4097, dtype=np.float64)
    assert remap_bucket(s).tolist() == list(range(4095)) + [4095, 4095]
    # degenerate ranges: one bucket
    assert remap_bucket(np.array([2.5, 2.5, 2.5])).tolist() == [0, 0, 0]
    assert remap_bucket(np.array([7.0])).tolist() == [0]
    assert remap_bucket(np.zeros(0)).tolist() == []
    # a span that overflows fp32 is no usable range either
    assert remap_bucket(np.array([-3e38, 3e38, 0.0])).tolist() == [0, 0, 0]


def test_remap_bucket_shift_scale_invariance_and_monotone():
    from oracle.method import remap_bucket
    rng = np.random.default_rng(52)
    s = rng.integers(-500, 500, 3000).astype(np.float64)
    b = remap_bucket(s)
    # exact integer arithmetic in fp32: shifting by an integer and scaling by
    # a power of two leave s - mn and span in the same ratio
    assert (remap_bucket(4.0 * s + 64.0) == b).all()
    assert (remap_bucket(s - 1000.0) == b).all()
    # non-decreasing, within range, ends pinned
    o = np.argsort(s, kind="stable")
    assert (np.diff(b[o]) >= 0).all()
    assert b.min() == 0 and b.max() == 4095
    assert b[np.argmin(s)] == 0 and b[np.argmax(s)] == 4095
    # a different bin count scales the grid: 2 bins split at the midpoint
    assert remap_bucket(np.array([0.0, 0.99, 1.0, 2.0]), bins=2).tolist() == [0, 0, 1, 1]


def test_approx_topk_hand_worked():
    from oracle.method import approx_select_tokens
    # buckets [0, 4095, 2048, 2048, 1024] (above): k = 2 keeps 4.0 (certain)
    # and fills one of the two units of bucket 2048 in index order; the exact
    # top-2 takes the larger score of that bucket instead
    s = np.array([0.0, 4.0, 2.0, 2.0005, 1.0])
    assert approx_select_tokens(s, 2) == [1, 2]
    assert select_tokens(s, 2) == [1, 3]
    assert approx_select_tokens(s, 3) == [1, 2, 3] == select_tokens(s, 3)
    assert approx_select_tokens(s, 5) == [0, 1, 2, 3, 4]
    assert approx_select_tokens(s, 0) == []
    # equal scores: one bucket, index order, as in the exact ranking
    assert approx_select_tokens(np.ones(6), 4) == [0, 1, 2, 3] == select_tokens(np.ones(6), 4)
    # candidates: the range is that of the candidates' scores
    c = [1, 3, 4]
    assert approx_select_tokens(s, 1, candidates=c) == [1]
    assert approx_select_tokens(s, 2, candidates=c) == [1, 3]


def test_approx_topk_exact_when_buckets_are_distinct():
    from oracle.method import approx_select_tokens, remap_bucket
    # scores 0, 1, ..., 4094 (span 4094 < 4096: every score its own bucket):
    # the approximate top-k is the exact one for every k
    rng = np.random.default_rng(50)
    s = rng.permutation(4095).astype(np.float64)
    assert len(set(remap_bucket(s).tolist())) == 4095
    for k in (0, 1, 7, 2048, 4095):
        assert approx_select_tokens(s, k) == select_tokens(s, k)


def test_approx_topk_keeps_every_certain_winner():
    from oracle.method import approx_select_tokens, remap_bucket
    rng = np.random.default_rng(51)
    s = rng.standard_normal(30000) * 5
    b = remap_bucket(s)
    for k in (10, 300, 2048, 29999):
        got = set(approx_select_tokens(s, k))
        exact = set(select_tokens(s, k))
        kth = np.sort(b)[::-1][k - 1]
        assert len(got) == k
        assert {i for i in range(len(s)) if b[i] > kth} <= got & exact
        assert all(b[i] >= kth for i in got)
        # only the boundary bucket can differ from the exact set
        assert len(got ^ exact) <= 2 * int((b == kth).sum())


# ------------------------------------------------------- sink + recent window

def test_window_tokens_cases():
    from oracle.method import window_tokens
    assert list(window_tokens(100, 4, 10)) == [0, 1, 2, 3] + list(range(90, 100))
    assert list(window_tokens(12, 4, 10)) == list(range(12))        # ranges touch
    assert list(window_tokens(3, 4, 10)) == [0, 1, 2]                # shorter than the sinks
    assert list(window_tokens(50, 0, 5)) == list(range(45, 50))
    assert list(window_tokens(50, 4, 0)) == [0, 1, 2, 3]
    assert list(window_tokens(0, 4, 10)) == []


def test_window_attention_is_the_lse_merge_of_two_calls():
    """The paper's form: the window and the sinks as two calls merged by
    log-sum-exp; equal to one softmax over the union."""
    from oracle.method import window_attention, window_tokens
    rng = np.random.default_rng(60)
    batch, npg = _tiny_batch(rng, lens=(37, 9))
    k = _rand_bf16(rng, (npg, 2, 4, 8))
    v = _rand_bf16(rng, (npg, 2, 4, 8))
    q = _rand_bf16(rng, (2, 4, 8))
    for r in range(2):
        L = int(batch.seq_lens[r])
        o, lse = window_attention(q, k, v, batch, r, 1, n_sink=3, window=20, num_kv_heads=2,
                                  sm_scale=0.3, out_dtype="fp64")
        t = window_tokens(L, 3, 20)
        sinks, win = t[t < 3], t[t >= 3]
        for i, h in enumerate((2, 3)):
            parts = []
            for part in (sinks, win):
                page, slot = batch.token_page_slot(r, part)
                K = bf16_to_f64(k[page, 1, slot])
                V = bf16_to_f64(v[page, 1, slot])
                parts.append(attention_over_tokens(bf16_to_f64(q[r, h]), K, V, 0.3))
            mo, ml = lse_merge(parts)
            np.testing.assert_allclose(o[i], mo, rtol=1e-12, atol=1e-14)
            assert abs(lse[i] - ml) <= 1e-12 * max(1.0, abs(ml))
        # a window covering everything is dense attention
        od, ld = dense_attention(q, k, v, batch, r, 1, num_kv_heads=2, sm_scale=0.3,
                                 out_dtype="fp64")
        ow, lw = window_attention(q, k, v, batch, r, 1, n_sink=0, window=L, num_kv_heads=2,
                                  sm_scale=0.3, out_dtype="fp64")
        np.testing.assert_allclose(ow, od, rtol=1e-12, atol=1e-14)


# ------------------------------------------------------ SnapKV-style selection

def test_snapkv_scores_sum_to_queries_times_heads_and_match_softmax():
    from oracle.method import snapkv_scores
    rng = np.random.default_rng(70)
    batch, npg = _tiny_batch(rng, lens=(30, 13))
    k = _rand_bf16(rng, (npg, 2, 4, 8))
    qo = _rand_bf16(rng, (2, 5, 4, 8))          # W = 5 observation queries, 4 q heads
    for r in range(2):
        L = int(batch.seq_lens[r])
        s = snapkv_scores(qo, k, batch, r, 1, num_kv_heads=2, sm_scale=0.4)
        assert abs(s.sum() - 5 * 2) < 1e-12                 # each softmax sums to 1
        # the last position is seen only by the last observation query
        # (its own position): p of one softmax per head
        t = np.arange(L)
        page, slot = batch.token_page_slot(r, t)
        K = bf16_to_f64(k[page, 1, slot])
        want_last = 0.0
        for h in (2, 3):
            # softmax weights of the last query via attention with one-hot values
            o, _ = attention_over_tokens(bf16_to_f64(qo[r, 4, h]), K, np.eye(L), 0.4)
            want_last += o[L - 1]
        assert abs(s[L - 1] - want_last) < 1e-12


def test_snapkv_select_pooling_and_forcing_hand_worked():
    from oracle.method import snapkv_select
    import oracle.method as om
    # scores by hand: a spike at prefix position 10 spreads to 7..13 after
    # the width-7 average, so with room for 7 ranked positions they are 7..13
    L, W = 40, 4
    batch = BatchView([0, 10], np.arange(10), [L], 4)
    fake = np.zeros(L)
    fake[10] = 7.0
    fake[30] = 0.5                     # a smaller bump far away
    orig = om.snapkv_scores
    om.snapkv_scores = lambda *a, **kw: fake
    try:
        qo = np.zeros((1, W, 1, 8), dtype=np.uint16)
        sel = snapkv_select(qo, None, batch, 0, 0, num_kv_heads=1, sm_scale=1.0, n_sink=2,
                            budget=2 + W + 7)
        assert sel == [0, 1] + list(range(7, 14)) + list(range(36, 40))
        # one more slot: the bump's neighbourhood (pooled 0.5/7) beats zeros,
        # the lowest of its 7 positions first
        sel = snapkv_select(qo, None, batch, 0, 0, num_kv_heads=1, sm_scale=1.0, n_sink=2,
                            budget=2 + W + 8)
        assert 27 in sel and 33 not in sel
        # a budget above L keeps everything
        assert snapkv_select(qo, None, batch, 0, 0, num_kv_heads=1, sm_scale=1.0, n_sink=2,
                             budget=100) == list(range(L))
    finally:
        om.snapkv_scores = orig


