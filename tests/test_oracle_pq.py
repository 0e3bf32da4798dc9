"""Pins for the oracle's PQ32 coarse scoring and two-pass selection
(LeanSparse §5, "Approximate scoring with PQ", Eq. 6).

Each test checks the oracle against something it does not share code with:
hand-worked k-means iterations and fixed-point means, nearest centroids found
with exact rationals, keys that are centroids, and the reductions of the
coarse score to the exact indexer score and of the two-pass selection to the
exact token top-k.
"""

from fractions import Fraction

import numpy as np

from oracle.method import BatchView, indexer_token_scores, select_tokens
from oracle.numerics import bf16_to_f64, f64_to_bf16_bits, fraction_to_bf16_bits
from oracle.pq import (dequantize_index_keys, fixed_point_mean_bf16, pq_decode, pq_encode,
                       pq_kmeans, pq_refine_select, pq_token_scores)


def test_fixed_point_mean_hand_worked():
    v = np.array([[1.0, 2.0, 3.0, 0.5], [2.0, 2.0, 2.0, 0.25], [1.0, 5.0, -1.0, 0.25]])
    got = bf16_to_f64(fixed_point_mean_bf16(v))
    # exact means 4/3, 3, 4/3, 1/3, each rounded once to bf16
    want = [fraction_to_bf16_bits(f) for f in (Fraction(4, 3), Fraction(3), Fraction(4, 3),
                                               Fraction(1, 3))]
    assert np.array_equal(fixed_point_mean_bf16(v), np.array(want, dtype=np.uint16))
    assert got[1] == 3.0
    # below the fixed-point unit: 2^-25 becomes rint(0.5) = 0 (half to even),
    # 3 * 2^-25 becomes rint(1.5) = 2 units of 2^-24
    tiny = np.array([[2.0 ** -25, 3 * 2.0 ** -25, 0.0, 0.0]] * 2)
    m = bf16_to_f64(fixed_point_mean_bf16(tiny))
    assert m[0] == 0.0 and m[1] == 2.0 ** -23


def test_encode_matches_exact_rational_argmin():
    rng = np.random.default_rng(40)
    cb = f64_to_bf16_bits(rng.standard_normal((32, 256, 4)))
    x = bf16_to_f64(f64_to_bf16_bits(rng.standard_normal((40, 128)) * 1.3))
    x[3, :4] = bf16_to_f64(cb[0, 17])           # a key subvector equal to a centroid
    cb[5, 9] = cb[5, 200]                        # a duplicated centroid: lowest index wins
    x[4, 20:24] = bf16_to_f64(cb[5, 200])
    codes = pq_encode(x, cb)
    cbq = [[[Fraction(float(v)) for v in c] for c in sub] for sub in bf16_to_f64(cb)]
    for i in range(x.shape[0]):
        for j in range(32):
            xs = [Fraction(float(v)) for v in x[i, 4 * j:4 * j + 4]]
            d = [sum((a - b) ** 2 for a, b in zip(xs, c)) for c in cbq[j]]
            assert codes[i, j] == int(np.argmin(np.array(d, dtype=object))) == d.index(min(d))
    assert codes[3, 0] == 17 and codes[4, 5] == 9


def test_kmeans_two_clusters_hand_worked():
    # five keys, every dim of a key equal: 0, 1, 2, 10, 11; centroids start
    # at keys 0 and 3. Iteration 1: {0, 1, 2} -> mean 1, {10, 11} -> 10.5;
    # iteration 2 changes nothing.
    vals = np.array([0.0, 1.0, 2.0, 10.0, 11.0])
    x = np.repeat(vals[:, None], 128, axis=1)
    for iters, want in ((1, (1.0, 10.5)), (2, (1.0, 10.5)), (0, (0.0, 10.0))):
        cb = bf16_to_f64(pq_kmeans(x, [0, 3], iters))
        assert cb.shape == (32, 2, 4)
        assert np.all(cb[:, 0] == want[0]) and np.all(cb[:, 1] == want[1])
    codes = pq_encode(x, pq_kmeans(x, [0, 3], 2))
    assert np.array_equal(codes, np.array([[0] * 32] * 3 + [[1] * 32] * 2))


def test_kmeans_empty_cluster_keeps_its_centroid():
    vals = np.array([0.0, 1.0, 3.0])
    x = np.repeat(vals[:, None], 128, axis=1)
    # centroids 0 and 1 both start at key 0: ties go to centroid 0, so
    # centroid 1 has no members and stays at 0; centroid 2 starts at key 2
    cb = bf16_to_f64(pq_kmeans(x, [0, 0, 2], 1))
    assert np.all(cb[:, 0] == 0.5) and np.all(cb[:, 1] == 0.0) and np.all(cb[:, 2] == 3.0)


def _tiny_pq_problem(rng, L=(150, 77), P=16):
    """Two requests over a permuted pool; fp8 keys with scale 1; a codebook
    holding every complete token's subvectors exactly (so codes are exact)."""
    nbs = [(n + P - 1) // P for n in L]
    npg = sum(nbs) + 2
    phys = rng.permutation(npg)[:sum(nbs)]
    batch = BatchView(np.concatenate([[0], np.cumsum(nbs)]), phys, np.array(L), P)
    # fp8 e4m3fn bits of small integers and halves (exact in bf16); each
    # subspace draws its subvectors from 200 of them
    table = rng.integers(-12, 13, size=(32, 200, 4)) / 2.0
    pick = rng.integers(0, 200, size=(npg * P, 32))
    vals = np.concatenate([table[j][pick[:, j]] for j in range(32)], axis=1).reshape(npg, P, 128)
    from oracle.numerics import fp8e4m3fn_to_f64
    codes8 = np.arange(256, dtype=np.uint8)
    dec = fp8e4m3fn_to_f64(codes8)
    lut = {float(v): int(c) for c, v in zip(codes8, dec) if np.isfinite(v) and c < 128}
    lut.update({float(v): int(c) for c, v in zip(codes8, dec) if np.isfinite(v) and c >= 128
                and float(v) not in lut})
    key_bits = np.vectorize(lambda v: lut[float(v)])(vals).astype(np.uint8)
    scales = np.ones((npg, P), dtype=np.float32)
    x = dequantize_index_keys(key_bits, scales).reshape(npg * P, 128)
    cb = np.full((32, 256, 4), 1000.0)
    for j in range(32):
        sub = np.unique(x[:, 4 * j:4 * j + 4], axis=0)
        assert len(sub) <= 256
        cb[j, :len(sub)] = sub
    cbb = f64_to_bf16_bits(cb)
    codes = pq_encode(x, cbb).reshape(npg, P, 32)
    return batch, key_bits, scales, codes, cbb, x


def test_coarse_score_is_the_exact_score_when_codes_are_exact():
    rng = np.random.default_rng(41)
    batch, key_bits, scales, codes, cb, x = _tiny_pq_problem(rng)
    assert np.array_equal(pq_decode(codes.reshape(-1, 32), cb), x)
    q = f64_to_bf16_bits(rng.standard_normal((2, 8, 128)))
    w = rng.standard_normal((2, 8)).astype(np.float32)
    for r in range(2):
        nc = batch.num_complete(r)
        t = np.arange(nc * batch.page_size)
        a = pq_token_scores(q, w, codes, cb, batch, r)
        b = indexer_token_scores(q, w, key_bits, scales, batch, r, tokens=t)
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_two_pass_selection_reduces_to_exact_topk():
    rng = np.random.default_rng(42)
    batch, key_bits, scales, codes, cb, _ = _tiny_pq_problem(rng)
    q = f64_to_bf16_bits(rng.standard_normal((2, 8, 128)))
    w = np.abs(rng.standard_normal((2, 8))).astype(np.float32)
    for r in range(2):
        L = int(batch.seq_lens[r])
        exact_all = indexer_token_scores(q, w, key_bits, scales, batch, r)
        want = select_tokens(exact_all, 10)
        # C covering every complete token: the exact top-k over all tokens
        res = pq_refine_select(q, w, key_bits, scales, codes, cb, batch, r,
                               n_candidates=L, topk=10)
        assert res["selected"] == want
        # exact codes and C >= k: the coarse pass keeps every complete token
        # of the exact top-k, so the result is the same
        res = pq_refine_select(q, w, key_bits, scales, codes, cb, batch, r,
                               n_candidates=12, topk=10)
        assert res["selected"] == want
        assert len(res["candidates"]) == 12
        assert list(res["refined"]) == sorted(res["refined"])


def test_two_pass_cannot_recover_a_token_the_coarse_pass_drops():
    # codes that all point at one centroid make every coarse score equal:
    # the candidates are the lowest tokens, and the selection lies inside
    # them plus the tail
    rng = np.random.default_rng(43)
    batch, key_bits, scales, codes, cb, _ = _tiny_pq_problem(rng)
    flat = np.zeros_like(codes)
    q = f64_to_bf16_bits(rng.standard_normal((2, 8, 128)))
    w = np.abs(rng.standard_normal((2, 8))).astype(np.float32)
    res = pq_refine_select(q, w, key_bits, scales, flat, cb, batch, 0, n_candidates=20, topk=5)
    assert res["candidates"] == list(range(20))
    tail = set(range(batch.num_complete(0) * 16, int(batch.seq_lens[0])))
    assert set(res["selected"]) <= set(range(20)) | tail


# ------------------------------------------------------------- miss filter

def test_miss_filter_hand_worked_sample_deviation_and_equality():
    from oracle.pq import pq_miss_filter
    # scores 6, 4, 2 (tokens 10, 11, 12), all misses, k = 1: s_(1) = 6; mean 4,
    # squared deviations 4 + 0 + 4 = 8, sample variance 8 / 2 = 4, sd = 2:
    # theta = 4. The score 4 equals theta and stays; 2 is dropped. (With the
    # population deviation sqrt(8/3) = 1.63, theta = 4.37 would drop 4 too;
    # with a strict "above theta", 4 would go.)
    r = pq_miss_filter([10, 11, 12], np.array([6.0, 4.0, 2.0]), np.zeros(3, bool), 1)
    assert r["theta"] == 4.0
    assert r["kept"] == [10, 11] and r["misses_kept"] == 2
    # a hit is kept whatever its score
    r = pq_miss_filter([10, 11, 12], np.array([6.0, 4.0, 2.0]), np.array([0, 0, 1], bool), 1)
    assert r["kept"] == [10, 11, 12] and r["misses_kept"] == 2


def test_miss_filter_hand_worked_kth_largest():
    from oracle.pq import pq_miss_filter
    # scores 1, 9, 5, 7, 4 (tokens 0..4), k = 1: s_(1) = 9; mean 5.2, squared
    # deviations 17.64 + 14.44 + 0.04 + 3.24 + 1.44 = 36.8, sample variance
    # 9.2, sd 3.0332: theta = 5.9668 keeps 9 and 7 only. (The k-th smallest,
    # 1, would keep everything; the (k+1)-th largest, 7, would keep 5 and 4.)
    s = np.array([1.0, 9.0, 5.0, 7.0, 4.0])
    r = pq_miss_filter(range(5), s, np.zeros(5, bool), 1)
    assert abs(r["theta"] - (9.0 - np.sqrt(9.2))) < 1e-12
    assert r["kept"] == [1, 3]
    # k = 3: s_(3) = 5, theta = 1.9668: only 1 is dropped
    assert pq_miss_filter(range(5), s, np.zeros(5, bool), 3)["kept"] == [1, 2, 3, 4]


def test_miss_filter_degenerate_sizes():
    from oracle.pq import pq_miss_filter
    # k >= n: s_(k) is the smallest score, theta <= every score: all kept
    s = np.array([3.0, -1.0, 8.0])
    assert pq_miss_filter([5, 6, 7], s, np.zeros(3, bool), 3)["kept"] == [5, 6, 7]
    assert pq_miss_filter([5, 6, 7], s, np.zeros(3, bool), 50)["kept"] == [5, 6, 7]
    # one candidate: sd = 0, theta = its score: kept
    assert pq_miss_filter([9], np.array([2.5]), np.zeros(1, bool), 1)["kept"] == [9]
    assert pq_miss_filter([], np.zeros(0), np.zeros(0, bool), 4)["kept"] == []
    # scores are taken as fp32: 0.1 and its fp32 rounding are the same score
    a = pq_miss_filter([0, 1], np.array([0.1, np.float32(0.1)]), np.zeros(2, bool), 1)
    assert a["theta"] == float(np.float32(0.1)) and a["kept"] == [0, 1]
