"""GPU parity of PQ32 coarse-to-fine indexing (LeanSparse §5, "Approximate
scoring with PQ" and "Retrieving and refining candidates"): k-means
codebooks and codes bit-exact against the oracle; coarse scores within 1e-5
of the oracle's (relative to the sum of absolute terms); candidate and final
selections exact outside the near-tie band.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from oracle.method import BatchView
from oracle.pq import dequantize_index_keys, pq_encode, pq_kmeans, pq_token_scores
from parity_util import TIE_ABS_OF_MAX, TIE_REL, say
from workloads import (PQ32_128K, bf16_bits, fp8_bits, make_indexer_inputs, pq_init_tokens,
                       reduced)

pytestmark = pytest.mark.gpu

ls = pytest.importorskip("query_aware_sparse_ls_amd")

SCORE_REL = 1e-5


def _dev():
    assert torch.cuda.is_available()
    return torch.device("cuda:0")


def _inputs(batch=2, blocks=40, lens=None, seed=11, page_size=64):
    cfg = reduced(PQ32_128K, batch=batch, context=blocks * page_size, seed=seed,
                  page_size=page_size)
    inp = make_indexer_inputs(cfg, device=_dev())
    if lens is not None:
        inp.seq_lens.copy_(torch.tensor(lens, dtype=torch.int32))
    return inp


def _batch(inp):
    P = inp.cfg.page_size
    nb = max(1, int((inp.seq_lens.max().item() + P - 1) // P))
    return ls.PagedBatch(inp.idx_indptr, inp.idx_indices, inp.seq_lens, nb)


def _train(inp, iters, n_pages=None):
    """Codebooks trained on the first n_pages pages of the pool (GPU)."""
    P = inp.cfg.page_size
    n_pages = n_pages or int(inp.idx_keys.shape[0])
    ids = torch.arange(n_pages, dtype=torch.int32, device=_dev())
    init = pq_init_tokens(n_pages * P, inp.cfg.seed).to(_dev())
    cb = ls.pq_train(inp.idx_keys, inp.idx_scale, ids, init, iters)
    return cb, ids, init


def _encode_all(inp, cb):
    n = int(inp.idx_keys.shape[0])
    codes = torch.zeros(n, inp.cfg.page_size, 32, dtype=torch.uint8, device=_dev())
    ids = torch.arange(n, dtype=torch.int32, device=_dev())
    ls.pq_encode(inp.idx_keys, inp.idx_scale, ids, cb, codes)
    return codes


def _host_keys(inp):
    return dequantize_index_keys(fp8_bits(inp.idx_keys), inp.idx_scale.cpu().numpy())


def _check_topk(gpu_sel, scores, cands, k, what):
    """gpu_sel (ascending ids) vs the oracle's top-k of `cands` by (score
    desc, id asc): exact outside the near-tie band around the k-th score."""
    want = oracle.select_tokens(scores, k, candidates=cands)
    assert gpu_sel == sorted(set(gpu_sel)), (what, "not ascending/unique")
    assert len(gpu_sel) == len(want), (what, len(gpu_sel), len(want))
    band = set()
    if 0 < k < len(cands):
        s = np.array([scores[j] for j in cands])
        sk = np.sort(s)[::-1][k - 1]
        tau = TIE_REL * abs(sk) + TIE_ABS_OF_MAX * np.max(np.abs(s))
        band = {j for j in cands if abs(scores[j] - sk) <= tau}
    diff = set(gpu_sel) ^ set(want)
    assert diff <= band, (what, sorted(diff)[:10], len(band))
    return len(band)


def test_pq_train_and_encode_bit_exact():
    """k-means (3 iterations over 40 pages x 64 tokens) and the codes of
    every page equal the oracle's, bit for bit."""
    inp = _inputs(batch=1, blocks=40, seed=21)
    cb, _, init = _train(inp, 3)
    codes = _encode_all(inp, cb)
    torch.cuda.synchronize()
    x = _host_keys(inp).reshape(-1, 128)
    want_cb = pq_kmeans(x, init.cpu().numpy(), 3)
    assert np.array_equal(bf16_bits(cb), want_cb)
    want_codes = pq_encode(x, want_cb).reshape(codes.shape)
    assert np.array_equal(codes.cpu().numpy(), want_codes)
    # zero iterations: the starting centroids
    cb0, _, _ = _train(inp, 0)
    assert np.array_equal(bf16_bits(cb0), pq_kmeans(x, init.cpu().numpy(), 0))


def test_pq_encode_listed_pages_only():
    """Only the listed pages' codes are written (duplicates allowed; ids out
    of range skipped); codebook random bf16."""
    inp = _inputs(batch=1, blocks=30, seed=22)
    g = torch.Generator().manual_seed(5)
    cb = torch.randn(32, 256, 4, generator=g).to(torch.bfloat16).to(_dev())
    n = int(inp.idx_keys.shape[0])
    ids = torch.tensor([3, 7, 7, 0, n - 1, -1, n + 5], dtype=torch.int32, device=_dev())
    codes = torch.full((n, 64, 32), 255, dtype=torch.uint8, device=_dev())
    ls.pq_encode(inp.idx_keys, inp.idx_scale, ids, cb, codes)
    torch.cuda.synchronize()
    got = codes.cpu().numpy()
    x = _host_keys(inp)
    listed = [3, 7, 0, n - 1]
    want = pq_encode(x[listed].reshape(-1, 128), bf16_bits(cb)).reshape(len(listed), 64, 32)
    assert np.array_equal(got[listed], want)
    others = np.setdiff1d(np.arange(n), listed)
    assert (got[others] == 255).all()


@pytest.mark.parametrize("lens,C", [((2500, 1300), 300), ((64, 3), 10), ((1000, 640), 5000),
                                    ((2560, 2000), 0)])
def test_pq_select_and_refine_small(lens, C):
    """Coarse scores, top-C candidates and the exact rerank (top-64 of the
    candidates and the partial page) against the oracle; lengths with no
    complete page, no partial page, and C above the number of tokens."""
    inp = _inputs(batch=2, blocks=40, lens=lens, seed=23)
    say(f"pq select: lens {lens}, C {C}")
    cb, _, _ = _train(inp, 2)
    codes = _encode_all(inp, cb)
    b = _batch(inp)
    P = inp.cfg.page_size
    stride = ls.indexer_score_stride("tokens", b.max_blocks * P)
    sc = torch.full((2, stride), float("nan"), device=_dev())
    cand, cnt = ls.pq_select(inp.q_idx, inp.head_w, codes, cb, b, C, scores_out=sc)
    k = 64
    ex_stride = ls.indexer_score_stride("tokens", max(C, 1) + P)
    esc = torch.full((2, ex_stride), float("nan"), device=_dev())
    sel, n = ls.indexer_select(inp.q_idx, inp.head_w, inp.idx_keys, P, b, granularity="tokens",
                               topk=k, max_selected=k, key_scales=inp.idx_scale,
                               cand_blocks=cand, cand_counts=cnt, token_candidates=True,
                               scores_out=esc)
    torch.cuda.synchronize()
    q, w = bf16_bits(inp.q_idx), inp.head_w.cpu().numpy()
    bv = BatchView(inp.idx_indptr.cpu().numpy(), inp.idx_indices.cpu().numpy(),
                   inp.seq_lens.cpu().numpy(), P)
    cbb = bf16_bits(cb)
    codes_h = codes.cpu().numpy()
    kb, ks = fp8_bits(inp.idx_keys), inp.idx_scale.cpu().numpy()
    for r in range(2):
        L = lens[r]
        nc = L // P
        coarse = pq_token_scores(q, w, codes_h, cbb, bv, r)
        # tolerance scale: the sum of absolute terms with the decoded keys
        dec = oracle.pq.pq_decode(codes_h[bv.pages(r)[:nc]].reshape(-1, 32), cbb)
        mag = (np.abs(dec) @ np.abs(oracle.bf16_to_f64(q[r])).T) @ np.abs(w[r].astype(np.float64))
        got = sc[r, :nc * P].cpu().numpy().astype(np.float64)
        assert np.all(np.abs(got - coarse) <= SCORE_REL * mag + 1e-30), "coarse scores"
        c_n = int(cnt[r])
        gc = cand[r, :c_n].cpu().tolist()
        _check_topk(gc, coarse, list(range(nc * P)), C, f"candidates r{r}")
        if C > c_n:
            assert (cand[r, c_n:] == -1).all()
        # the exact pass scores the GPU's candidates and the tail
        refined = np.array(gc + list(range(nc * P, L)), dtype=np.int64)
        exact = oracle.indexer_token_scores(q, w, kb, ks, bv, r, tokens=refined)
        gx = esc[r, :len(refined)].cpu().numpy().astype(np.float64)
        np.testing.assert_allclose(gx, exact, rtol=2e-5,
                                   atol=1e-5 * max(1.0, np.abs(exact).max(initial=0.0)))
        pos = {t: i for i, t in enumerate(refined.tolist())}
        gsel = sorted(pos[t] for t in sel[r, :int(n[r])].cpu().tolist())
        _check_topk(gsel, exact, list(range(len(refined))), k, f"final r{r}")
        assert (sel[r, int(n[r]):] == -1).all()


def test_pq_full_size_sampled():
    """The bench shape (8 x 128K, 64 heads, C = 2,048, k = 512), codebooks
    trained on the cache: requests 0 and 7 against the oracle."""
    cfg = PQ32_128K
    say(f"pq at full size: {cfg.name}")
    inp = make_indexer_inputs(cfg, device=_dev())
    P = cfg.page_size
    cb, _, _ = _train(inp, 2)
    codes = _encode_all(inp, cb)
    b = _batch(inp)
    stride = ls.indexer_score_stride("tokens", b.max_blocks * P)
    sc = torch.empty((cfg.batch, stride), device=_dev())
    cand, cnt = ls.pq_select(inp.q_idx, inp.head_w, codes, cb, b, cfg.n_candidates, scores_out=sc)
    sel, n = ls.indexer_select(inp.q_idx, inp.head_w, inp.idx_keys, P, b, granularity="tokens",
                               topk=cfg.topk_tokens, max_selected=cfg.topk_tokens,
                               key_scales=inp.idx_scale, cand_blocks=cand, cand_counts=cnt,
                               token_candidates=True)
    torch.cuda.synchronize()
    q, w = bf16_bits(inp.q_idx), inp.head_w.cpu().numpy()
    bv = BatchView(inp.idx_indptr.cpu().numpy(), inp.idx_indices.cpu().numpy(),
                   inp.seq_lens.cpu().numpy(), P)
    cbb, codes_h = bf16_bits(cb), codes.cpu().numpy()
    kb, ks = fp8_bits(inp.idx_keys), inp.idx_scale.cpu().numpy()
    for r in (0, 7):
        coarse = pq_token_scores(q, w, codes_h, cbb, bv, r)
        gc = cand[r, :int(cnt[r])].cpu().tolist()
        _check_topk(gc, coarse, list(range(len(coarse))), cfg.n_candidates, f"candidates r{r}")
        exact = oracle.indexer_token_scores(q, w, kb, ks, bv, r, tokens=np.array(gc))
        pos = {t: i for i, t in enumerate(gc)}
        gsel = [pos[t] for t in sel[r, :int(n[r])].cpu().tolist()]
        _check_topk(sorted(gsel), exact, list(range(len(gc))), cfg.topk_tokens, f"final r{r}")


@pytest.mark.parametrize("page_size", [16, 32])
def test_pq_small_pages(page_size):
    """16- and 32-token pages: codes, candidates and the exact rerank against
    the oracle (ragged lengths with a partial page)."""
    lens = (150 * page_size + 5, 37 * page_size)
    inp = _inputs(batch=2, blocks=160, lens=lens, seed=31 + page_size, page_size=page_size)
    P = page_size
    cb, _, _ = _train(inp, 1)
    codes = _encode_all(inp, cb)
    b = _batch(inp)
    C, k = 700, 100
    cand, cnt = ls.pq_select(inp.q_idx, inp.head_w, codes, cb, b, C)
    sel, n = ls.indexer_select(inp.q_idx, inp.head_w, inp.idx_keys, P, b, granularity="tokens",
                               topk=k, max_selected=k, key_scales=inp.idx_scale,
                               cand_blocks=cand, cand_counts=cnt, token_candidates=True)
    torch.cuda.synchronize()
    q, w = bf16_bits(inp.q_idx), inp.head_w.cpu().numpy()
    bv = BatchView(inp.idx_indptr.cpu().numpy(), inp.idx_indices.cpu().numpy(),
                   inp.seq_lens.cpu().numpy(), P)
    x = _host_keys(inp).reshape(-1, 128)
    assert np.array_equal(codes.cpu().numpy().reshape(-1, 32), pq_encode(x, bf16_bits(cb)))
    kb, ks = fp8_bits(inp.idx_keys), inp.idx_scale.cpu().numpy()
    for r, L in enumerate(lens):
        nc = L // P
        coarse = pq_token_scores(q, w, codes.cpu().numpy(), bf16_bits(cb), bv, r)
        gc = cand[r, :int(cnt[r])].cpu().tolist()
        _check_topk(gc, coarse, list(range(nc * P)), C, f"candidates r{r}")
        refined = np.array(gc + list(range(nc * P, L)), dtype=np.int64)
        exact = oracle.indexer_token_scores(q, w, kb, ks, bv, r, tokens=refined)
        pos = {t: i for i, t in enumerate(refined.tolist())}
        gsel = sorted(pos[t] for t in sel[r, :int(n[r])].cpu().tolist())
        _check_topk(gsel, exact, list(range(len(refined))), k, f"final r{r}")


# ------------------------------------------------------------- miss filter

def _resident_bits(B, n_tokens, rate, seed):
    """Seeded residency flags [B][n_tokens] and their bitmap [B][words] int32."""
    g = np.random.default_rng(seed)
    flags = g.random((B, n_tokens)) < rate
    words = (n_tokens + 31) // 32
    bits = np.zeros((B, words * 32), dtype=bool)
    bits[:, :n_tokens] = flags
    w = (bits.reshape(B, words, 32).astype(np.uint64) << np.arange(32, dtype=np.uint64)).sum(-1)
    return flags, torch.from_numpy(w.astype(np.uint32).view(np.int32)).to(_dev())


def test_miss_filter_hand_worked():
    """Scores 6, 4, 2 (tokens 10 .. 12), k = 1: theta = 6 - 2 = 4 exactly; the
    miss at 4 stays, the miss at 2 goes unless it is resident."""
    cand = torch.tensor([[10, 11, 12, -1], [10, 11, 12, -1]], dtype=torch.int32, device=_dev())
    cnt = torch.tensor([3, 3], dtype=torch.int32, device=_dev())
    sc = torch.zeros(2, 16, device=_dev())
    sc[:, 10:13] = torch.tensor([6.0, 4.0, 2.0])
    res = torch.zeros(2, 1, dtype=torch.int32, device=_dev())
    res[1, 0] = 1 << 12
    kept, kn, mk = ls.pq_filter_misses(cand, cnt, sc, res, 1)
    torch.cuda.synchronize()
    assert kept[0].tolist() == [10, 11, -1, -1] and int(kn[0]) == 2 and int(mk[0]) == 2
    assert kept[1].tolist() == [10, 11, 12, -1] and int(kn[1]) == 3 and int(mk[1]) == 2


@pytest.mark.parametrize("inplace", [False, True])
def test_miss_filter_parity_synthetic(inplace):
    """Seeded candidates (ascending tokens), fp32 scores and residency (40%
    hits) for requests of 2,048, 1,000, 1, 0 and 4,096 (the cap) candidates
    with k = 512, against the oracle; only candidates within 1e-9 of theta
    (where the two float64 sum orders could disagree) are excused."""
    B, cap, stride, k = 5, 4096, 20000, 512
    counts = [2048, 1000, 1, 0, 4096]
    g = np.random.default_rng(91)
    cand = np.full((B, cap), -1, dtype=np.int32)
    for r, c in enumerate(counts):
        cand[r, :c] = np.sort(g.choice(stride, size=c, replace=False))
    scores = (g.standard_normal((B, stride)) * 7 + 3).astype(np.float32)
    flags, res = _resident_bits(B, stride, 0.4, 92)
    say(f"miss filter synthetic, inplace {inplace}")
    cand_d = torch.from_numpy(cand).to(_dev())
    cnt_d = torch.tensor(counts, dtype=torch.int32, device=_dev())
    sc_d = torch.from_numpy(scores).to(_dev())
    kept, kn, mk = ls.pq_filter_misses(cand_d, cnt_d, sc_d, res, k,
                                       kept=cand_d if inplace else None)
    torch.cuda.synchronize()
    kept, kn, mk = kept.cpu().numpy(), kn.cpu().numpy(), mk.cpu().numpy()
    for r, c in enumerate(counts):
        t = cand[r, :c]
        want = oracle.pq.pq_miss_filter(t, scores[r, t], flags[r, t], k)
        got = kept[r, :kn[r]].tolist()
        assert (kept[r, kn[r]:] == -1).all()
        near = {int(x) for x in t if abs(float(scores[r, x]) - want["theta"]) <= 1e-9 * max(1.0, abs(want["theta"]))}
        assert set(got) ^ set(want["kept"]) <= near, r
        assert got == sorted(got)
        if not near:
            assert got == want["kept"] and int(mk[r]) == want["misses_kept"]


def test_miss_filter_in_the_pq_pipeline_full_size():
    """The bench shape (8 x 128K, C = 2,048, k = 512): PQ candidates, the miss
    filter with seeded residency (50% hits), then the exact rerank of the kept
    candidates; requests 0 and 7 against the oracle's filter on the oracle's
    coarse scores of those candidates (near theta, within the coarse scores'
    tolerance, either decision is accepted)."""
    cfg = PQ32_128K
    say(f"pq + miss filter at full size: {cfg.name}")
    inp = make_indexer_inputs(cfg, device=_dev())
    P = cfg.page_size
    cb, _, _ = _train(inp, 2)
    codes = _encode_all(inp, cb)
    b = _batch(inp)
    stride = ls.indexer_score_stride("tokens", b.max_blocks * P)
    sc = torch.empty((cfg.batch, stride), device=_dev())
    cand, cnt = ls.pq_select(inp.q_idx, inp.head_w, codes, cb, b, cfg.n_candidates, scores_out=sc)
    flags, res = _resident_bits(cfg.batch, b.max_blocks * P, 0.5, 93)
    kept, kn, mk = ls.pq_filter_misses(cand, cnt, sc, res, cfg.topk_tokens)
    sel, n = ls.indexer_select(inp.q_idx, inp.head_w, inp.idx_keys, P, b, granularity="tokens",
                               topk=cfg.topk_tokens, max_selected=cfg.topk_tokens,
                               key_scales=inp.idx_scale, cand_blocks=kept, cand_counts=kn,
                               token_candidates=True)
    torch.cuda.synchronize()
    q, w = bf16_bits(inp.q_idx), inp.head_w.cpu().numpy()
    bv = BatchView(inp.idx_indptr.cpu().numpy(), inp.idx_indices.cpu().numpy(),
                   inp.seq_lens.cpu().numpy(), P)
    cbb, codes_h = bf16_bits(cb), codes.cpu().numpy()
    kb, ks = fp8_bits(inp.idx_keys), inp.idx_scale.cpu().numpy()
    for r in (0, 7):
        coarse = pq_token_scores(q, w, codes_h, cbb, bv, r)
        gc = cand[r, :int(cnt[r])].cpu().tolist()
        _check_topk(gc, coarse, list(range(len(coarse))), cfg.n_candidates, f"candidates r{r}")
        t = np.array(gc)
        want = oracle.pq.pq_miss_filter(t, coarse[t], flags[r, t], cfg.topk_tokens)
        got = kept[r, :int(kn[r])].cpu().tolist()
        tol = 1e-4 * np.abs(coarse[t]).max()
        near = {int(x) for x in t if abs(coarse[x] - want["theta"]) <= tol}
        assert set(got) ^ set(want["kept"]) <= near, r
        dropped = len(gc) - len(got)
        say(f"request {r}: {len(gc)} candidates, {int((~flags[r, t]).sum())} misses, "
            f"{dropped} dropped, {int(mk[r])} misses kept")
        assert dropped > 0
        # the rerank over the kept candidates (and the partial page)
        exact = oracle.indexer_token_scores(q, w, kb, ks, bv, r, tokens=np.array(got))
        pos = {x: i for i, x in enumerate(got)}
        gsel = [pos[x] for x in sel[r, :int(n[r])].cpu().tolist()]
        _check_topk(sorted(gsel), exact, list(range(len(got))), cfg.topk_tokens, f"final r{r}")
