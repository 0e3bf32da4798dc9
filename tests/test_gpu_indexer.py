"""GPU parity of the learned-indexer selection (tokens and blocks), the sparse
MLA attention and their coarse-to-fine composition, through the C ABI,
against the float64 oracle on the same input bits.

Tolerances: indexer scores within 1e-5 of the sum of the magnitudes of their
terms (fp32 accumulation of exact products); selections exact outside the
near-tie band (1e-4 relative of the k-th score, + 1e-6 of the largest);
attention outputs within 2e-2 (bf16) / 1e-5 (fp32) absolute.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from oracle.method import BatchView
from parity_util import BF16_ATOL, FP32_ATOL, TIE_ABS_OF_MAX, TIE_REL, say
from workloads import (COARSE_TO_FINE_950K, INDEXER_128K, bf16_bits, fp8_bits,
                       make_indexer_inputs, reduced)

pytestmark = pytest.mark.gpu

ls = pytest.importorskip("query_aware_sparse_ls_amd")

SCORE_REL = 1e-5


def _dev():
    assert torch.cuda.is_available()
    return torch.device("cuda:0")


def _host(inp):
    """Host bit copies of the indexer inputs, and the two page tables."""
    P = inp.cfg.page_size
    h = dict(q=bf16_bits(inp.q_idx), w=inp.head_w.cpu().numpy(), k=fp8_bits(inp.idx_keys),
             s=inp.idx_scale.cpu().numpy(), lens=inp.seq_lens.cpu().numpy())
    h["ib"] = BatchView(inp.idx_indptr.cpu().numpy(), inp.idx_indices.cpu().numpy(), h["lens"], P)
    h["kb"] = BatchView(inp.kv_indptr.cpu().numpy(), inp.kv_indices.cpu().numpy(), h["lens"], P)
    return h


def _batch(inp, kv=False):
    P = inp.cfg.page_size
    nb = int((inp.seq_lens.max().item() + P - 1) // P)
    nb = max(nb, 1)
    if kv:
        return ls.PagedBatch(inp.kv_indptr, inp.kv_indices, inp.seq_lens, nb)
    return ls.PagedBatch(inp.idx_indptr, inp.idx_indices, inp.seq_lens, nb)


def _score_mag(h, r, tokens):
    """Sum over heads of |w_h| * sum_d |q_hd sigma k_d| (tolerance scale)."""
    page, slot = h["ib"].token_page_slot(r, np.asarray(tokens))
    k = np.abs(oracle.numerics.fp8e4m3fn_to_f64(h["k"][page, slot])) * \
        np.abs(h["s"][page, slot].astype(np.float64))[:, None]
    q = np.abs(oracle.numerics.bf16_to_f64(h["q"][r]))
    return (k @ q.T) @ np.abs(h["w"][r].astype(np.float64))


def _check_scores(got, want, mag, what):
    err = np.abs(got.astype(np.float64) - want)
    bad = err > SCORE_REL * mag + 1e-30
    assert not bad.any(), (what, int(bad.sum()), float((err / (mag + 1e-30)).max()))


def _check_topk(gpu_sel, scores, cands, k, what):
    """gpu_sel (ascending ids) vs the oracle's top-k of `cands` by (score desc,
    id asc): exact outside the near-tie band around the k-th score."""
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


def _small_indexer(batch=2, blocks=80, lens=None, seed=7, page_size=64, heads=64):
    cfg = reduced(INDEXER_128K, batch=batch, context=blocks * page_size, page_size=page_size,
                  index_heads=heads, seed=seed)
    inp = make_indexer_inputs(cfg, device=_dev())
    if lens is not None:
        inp.seq_lens.copy_(torch.tensor(lens, dtype=torch.int32))
    return inp


def _run_tokens(inp, topk, max_selected=None, cand=None, cnt=None):
    P = inp.cfg.page_size
    b = _batch(inp)
    max_selected = max_selected or max(topk, 1)
    units = (cand.shape[1] if cand is not None else b.max_blocks) * P
    stride = ls.indexer_score_stride("tokens", units)
    sc = torch.full((inp.cfg.batch, stride), float("nan"), device=_dev())
    sel, n = ls.indexer_select(inp.q_idx, inp.head_w, inp.idx_keys, P, b, granularity="tokens",
                               topk=topk, max_selected=max_selected, key_scales=inp.idx_scale,
                               cand_blocks=cand, cand_counts=cnt, scores_out=sc)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), n.cpu().numpy(), sc.cpu().numpy()


@pytest.mark.parametrize("lens,topk", [((5000, 3001), 256), ((1, 17), 4), ((4096, 64), 4096),
                                       ((777, 130), 0), ((5120, 2500), 2048)])
def test_indexer_token_topk_small(lens, topk):
    say(f"indexer tokens lens={lens} topk={topk}")
    inp = _small_indexer(lens=list(lens))
    h = _host(inp)
    sel, n, sc = _run_tokens(inp, topk, max_selected=max(topk, 1) + 3)
    for r, L in enumerate(lens):
        s = oracle.indexer_token_scores(h["q"], h["w"], h["k"], h["s"], h["ib"], r)
        _check_scores(sc[r, :L], s, _score_mag(h, r, np.arange(L)), f"scores r{r}")
        got = [int(x) for x in sel[r, :n[r]]]
        band = _check_topk(got, s, list(range(L)), topk, f"sel r{r}")
        assert np.all(sel[r, n[r]:] == -1)
        say(f"  r{r}: L={L} selected {n[r]} band {band}")


@pytest.mark.parametrize("L", [5000, 20000])
def test_indexer_all_equal_scores_take_lowest_tokens(L):
    """Zero keys give every token the score 0: the lowest token ids win. At
    L = 20000 the tied bucket exceeds the LDS candidate capacity and the
    ranking streams the scores instead."""
    say(f"indexer ties L={L}")
    inp = _small_indexer(batch=1, blocks=(L + 63) // 64, lens=[L])
    inp.idx_keys.view(torch.uint8).zero_()
    sel, n, sc = _run_tokens(inp, 300)
    assert n[0] == 300
    assert sel[0, :300].tolist() == list(range(300))
    assert np.all(sc[0, :L] == 0.0)


def test_indexer_candidate_blocks_and_block_mode():
    """Block mode on block-mean keys (forced recent block) feeding the token
    mode restricted to the kept blocks (the coarse-to-fine composition)."""
    say("indexer blocks + candidates")
    lens = [64 * 40, 64 * 37 + 20]
    inp = _small_indexer(batch=2, blocks=40, lens=lens, seed=11)
    h = _host(inp)
    P = inp.cfg.page_size
    b = _batch(inp)
    npg = inp.idx_keys.shape[0]
    summ = torch.zeros(npg, 128, dtype=torch.bfloat16, device=_dev())
    ls.build_block_summaries(inp.idx_keys, torch.arange(npg, dtype=torch.int32, device=_dev()),
                             summ, key_scales=inp.idx_scale)
    kb, kt = 8, 100
    bsc = torch.zeros(2, b.max_blocks, device=_dev())
    bsel, bn = ls.indexer_select(inp.q_idx, inp.head_w, summ, P, b, granularity="blocks",
                                 topk=kb, n_recent=1, max_selected=kb + 2, scores_out=bsc)
    tsel, tn = ls.indexer_select(inp.q_idx, inp.head_w, inp.idx_keys, P, b,
                                 granularity="tokens", topk=kt, max_selected=kt,
                                 key_scales=inp.idx_scale, cand_blocks=bsel, cand_counts=bn)
    torch.cuda.synchronize()
    summ_o = oracle.block_summaries(h["k"], range(npg), key_format="fp8_e4m3fn",
                                    key_scales=h["s"])
    assert np.array_equal(bf16_bits(summ), summ_o), "fp8 block means differ"
    for r in range(2):
        res = oracle.coarse_to_fine_select(h["q"], h["w"], h["k"], h["s"], summ_o, h["ib"], r,
                                           topk_blocks=kb, n_recent_blocks=1, topk_tokens=kt)
        nb, nc = h["ib"].num_blocks(r), h["ib"].num_complete(r)
        gb = [int(x) for x in bsel[r, :bn[r]].cpu()]
        forced = set(oracle.method.forced_blocks(nb, nc, 0, 1))
        cands = [j for j in range(nc) if j not in forced]
        sbs = np.full(nb, -np.inf)
        sbs[:nc] = res["block_scores"]
        got_b = bsc[r, :nb].cpu().numpy()
        assert np.allclose(got_b[cands], sbs[cands], rtol=1e-4, atol=1e-4)
        if gb != res["blocks"]:
            # only near-ties may differ; then the token stage is compared on
            # the GPU's own blocks
            _check_topk(sorted(set(gb) - forced), sbs, cands, kb, f"blocks r{r}")
            res = oracle.coarse_to_fine_select(h["q"], h["w"], h["k"], h["s"], summ_o, h["ib"],
                                               r, topk_blocks=nb, n_recent_blocks=1,
                                               topk_tokens=kt)
            toks = oracle.tokens_of_blocks(gb, P, lens[r])
            st = oracle.indexer_token_scores(h["q"], h["w"], h["k"], h["s"], h["ib"], r,
                                             tokens=toks)
            full = np.full(lens[r], -np.inf)
            full[toks] = st
            _check_topk([int(x) for x in tsel[r, :tn[r]].cpu()], full, toks.tolist(), kt,
                        f"tokens r{r}")
            continue
        full = np.full(lens[r], -np.inf)
        for t, v in res["token_scores"].items():
            full[t] = v
        band = _check_topk([int(x) for x in tsel[r, :tn[r]].cpu()], full,
                           sorted(res["token_scores"]), kt, f"tokens r{r}")
        say(f"  r{r}: blocks {len(gb)} tokens {int(tn[r])} band {band}")


def test_indexer_full_size_128k():
    """8 requests x 131,072 tokens, 64 heads, top-2048: scores on a sample of
    tokens of every request, the whole selection of requests 0 and 7."""
    say("indexer full size")
    inp = make_indexer_inputs(INDEXER_128K, device=_dev())
    h = _host(inp)
    cfg = INDEXER_128K
    sel, n, sc = _run_tokens(inp, cfg.topk_tokens)
    rng = np.random.default_rng(5)
    for r in range(cfg.batch):
        assert n[r] == cfg.topk_tokens
        t = np.sort(rng.choice(cfg.context, 512, replace=False))
        s = oracle.indexer_token_scores(h["q"], h["w"], h["k"], h["s"], h["ib"], r, tokens=t)
        _check_scores(sc[r, t], s, _score_mag(h, r, t), f"scores r{r}")
    for r in (0, cfg.batch - 1):
        s = oracle.indexer_token_scores(h["q"], h["w"], h["k"], h["s"], h["ib"], r)
        band = _check_topk([int(x) for x in sel[r, :n[r]]], s, list(range(cfg.context)),
                           cfg.topk_tokens, f"sel r{r}")
        say(f"  r{r}: band {band}")


# ------------------------------------------------------------------- MLA

def _run_mla(inp, sel, cnt, out_dtype, sm_scale):
    b = _batch(inp, kv=True)
    lse = torch.empty(inp.cfg.batch, inp.cfg.mla_heads, device=_dev())
    out, _ = ls.sparse_mla_decode(inp.q_mla, inp.latent, b, sel, cnt, sm_scale=sm_scale,
                                  out_dtype=out_dtype, lse=lse)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu().numpy()


def _check_mla(inp, h, out, lse, r, tokens, out_dtype, sm_scale, what):
    qb, lat = bf16_bits(inp.q_mla), None
    page, slot = h["kb"].token_page_slot(r, np.asarray(tokens, dtype=np.int64))
    # only the rows of the attended tokens are copied to the host
    rows = inp.latent.view(-1, 576)[torch.as_tensor(page * inp.cfg.page_size + slot,
                                                    device=inp.latent.device).long()]
    lat = bf16_bits(rows.contiguous()).reshape(-1, 1, 576)
    bv = BatchView(np.array([0, len(tokens)]), np.arange(len(tokens)), np.array([len(tokens)]), 1)
    o, l = oracle.mla_attention(qb[r:r + 1], lat, bv, 0, np.arange(len(tokens)), v_dim=512,
                                sm_scale=sm_scale,
                                out_dtype="fp32" if out_dtype == torch.float32 else "bf16")
    if out_dtype == torch.float32:
        got = out[r].numpy().astype(np.float64)
        err = np.abs(got - o.astype(np.float64)).max()
        assert err <= FP32_ATOL, (what, err)
    else:
        got = out[r].float().numpy().astype(np.float64)
        want = oracle.numerics.bf16_to_f64(o)
        err = np.abs(got - want).max()
        assert err <= BF16_ATOL, (what, err)
    if len(tokens):
        assert np.abs(lse[r] - l).max() <= 1e-4, what
    else:
        assert np.all(np.isneginf(lse[r])), what
    return err


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_mla_small_selected(out_dtype):
    say(f"mla small {out_dtype}")
    cfg = reduced(INDEXER_128K, batch=3, context=64 * 50, mla_heads=32, seed=21)
    inp = make_indexer_inputs(cfg, device=_dev())
    inp.seq_lens.copy_(torch.tensor([3200, 1000, 45], dtype=torch.int32))
    h = _host(inp)
    rng = np.random.default_rng(3)
    maxsel = 700
    sel = np.full((3, maxsel), -1, dtype=np.int32)
    cnt = np.zeros(3, dtype=np.int32)
    want_tokens = []
    for r, (L, k) in enumerate([(3200, 700), (1000, 333), (45, 0)]):
        t = np.sort(rng.choice(L, k, replace=False)) if k else np.zeros(0, dtype=np.int64)
        sel[r, :k] = t
        cnt[r] = k
        want_tokens.append(t)
    # an out-of-range id (>= L) is skipped
    sel[1, 332] = 5000
    want_tokens[1] = want_tokens[1][:332]
    sm = 1.0 / math.sqrt(576)
    out, lse = _run_mla(inp, torch.tensor(sel, device=_dev()), torch.tensor(cnt, device=_dev()),
                        out_dtype, sm)
    for r in range(3):
        err = _check_mla(inp, h, out, lse, r, want_tokens[r], out_dtype, sm, f"r{r}")
        say(f"  r{r}: {len(want_tokens[r])} tokens, max err {err:.2e}")


def test_mla_workspace_reused():
    """One workspace serves consecutive calls of different sizes and dtypes
    (the partial states of a call never leak into the next): each result is
    bit-identical to a call on a fresh workspace."""
    say("mla workspace reuse")
    cfg = reduced(INDEXER_128K, batch=3, context=64 * 50, mla_heads=64, seed=24)
    inp = make_indexer_inputs(cfg, device=_dev())
    inp.seq_lens.copy_(torch.tensor([3200, 2000, 700], dtype=torch.int32))
    b = _batch(inp, kv=True)
    rng = np.random.default_rng(5)
    maxsel = 1100
    sm = 1.0 / math.sqrt(576)
    ws = torch.full((ls.sparse_mla_decode_workspace_size(3, 64, maxsel),), 0xA5,
                    dtype=torch.uint8, device=_dev())   # need not be initialised
    for it, (ks, dt) in enumerate([((1100, 900, 700), torch.bfloat16),
                                   ((300, 1100, 5), torch.float32),
                                   ((1000, 0, 257), torch.bfloat16)]):
        sel = np.full((3, maxsel), -1, dtype=np.int32)
        for r, (L, k) in enumerate(zip([3200, 2000, 700], ks)):
            sel[r, :k] = np.sort(rng.choice(L, k, replace=False))
        sd = torch.tensor(sel, device=_dev())
        cd = torch.tensor(ks, dtype=torch.int32, device=_dev())
        out, _ = ls.sparse_mla_decode(inp.q_mla, inp.latent, b, sd, cd, sm_scale=sm,
                                      out_dtype=dt, workspace=ws)
        ref, _ = ls.sparse_mla_decode(inp.q_mla, inp.latent, b, sd, cd, sm_scale=sm,
                                      out_dtype=dt)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16) if dt == torch.bfloat16 else out.view(torch.int32),
                           ref.view(torch.int16) if dt == torch.bfloat16 else ref.view(torch.int32)), it


def test_mla_dense_equals_all_tokens():
    say("mla dense")
    cfg = reduced(INDEXER_128K, batch=2, context=64 * 9, mla_heads=32, seed=22)
    inp = make_indexer_inputs(cfg, device=_dev())
    inp.seq_lens.copy_(torch.tensor([576, 300], dtype=torch.int32))
    h = _host(inp)
    sm = 0.05
    out, lse = _run_mla(inp, None, None, torch.float32, sm)
    for r, L in enumerate([576, 300]):
        _check_mla(inp, h, out, lse, r, np.arange(L), torch.float32, sm, f"dense r{r}")


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_mla_dense_many_splits(out_dtype):
    """Every token of a 4,160-token cache: 17 splits of 256 tokens, so the
    merge takes three rounds of eight splits, the last one padded; requests
    shorter than the cache leave trailing splits empty."""
    say(f"mla dense, 17 splits, out {out_dtype}")
    lens = [4160, 2305, 1]
    cfg = reduced(INDEXER_128K, batch=3, context=64 * 65, mla_heads=32, seed=27)
    inp = make_indexer_inputs(cfg, device=_dev())
    inp.seq_lens.copy_(torch.tensor(lens, dtype=torch.int32))
    h = _host(inp)
    sm = 0.05
    out, lse = _run_mla(inp, None, None, out_dtype, sm)
    for r, L in enumerate(lens):
        _check_mla(inp, h, out, lse, r, np.arange(L), out_dtype, sm, f"dense r{r} L{L}")


def test_mla_full_size_config4():
    """8 requests x 2,048 selected tokens of 131,072, 128 heads, bf16 out:
    every head of requests 0 and 7 against the oracle."""
    say("mla full size")
    cfg = INDEXER_128K
    inp = make_indexer_inputs(cfg, device=_dev())
    h = _host(inp)
    rng = np.random.default_rng(9)
    sel = np.stack([np.sort(rng.choice(cfg.context, cfg.topk_tokens, replace=False))
                    for _ in range(cfg.batch)]).astype(np.int32)
    cnt = np.full(cfg.batch, cfg.topk_tokens, dtype=np.int32)
    sm = 1.0 / math.sqrt(576)
    out, lse = _run_mla(inp, torch.tensor(sel, device=_dev()), torch.tensor(cnt, device=_dev()),
                        torch.bfloat16, sm)
    for r in (0, cfg.batch - 1):
        err = _check_mla(inp, h, out, lse, r, sel[r], torch.bfloat16, sm, f"r{r}")
        say(f"  r{r}: max err {err:.2e}")


def test_coarse_to_fine_full_pipeline_reduced():
    """Config-5 pipeline at reduced length: fp8 block means, coarse block
    top-256 + last block, exact token top-2048 among their tokens, sparse
    MLA over them; compared step by step with the oracle."""
    say("coarse-to-fine reduced")
    cfg = reduced(COARSE_TO_FINE_950K, batch=2, context=64 * 600, mla_heads=32, seed=33)
    inp = make_indexer_inputs(cfg, device=_dev())
    h = _host(inp)
    P = cfg.page_size
    b = _batch(inp)
    npg = inp.idx_keys.shape[0]
    summ = torch.zeros(npg, 128, dtype=torch.bfloat16, device=_dev())
    ls.build_block_summaries(inp.idx_keys, torch.arange(npg, dtype=torch.int32, device=_dev()),
                             summ, key_scales=inp.idx_scale)
    kb, kt = cfg.coarse_topk_blocks, cfg.topk_tokens
    bsel, bn = ls.indexer_select(inp.q_idx, inp.head_w, summ, P, b, granularity="blocks",
                                 topk=kb, n_recent=1, max_selected=kb + 2)
    tsel, tn = ls.indexer_select(inp.q_idx, inp.head_w, inp.idx_keys, P, b,
                                 granularity="tokens", topk=kt, max_selected=kt,
                                 key_scales=inp.idx_scale, cand_blocks=bsel, cand_counts=bn)
    sm = 1.0 / math.sqrt(576)
    out, lse = _run_mla(inp, tsel, tn, torch.bfloat16, sm)
    summ_o = oracle.block_summaries(h["k"], range(npg), key_format="fp8_e4m3fn",
                                    key_scales=h["s"])
    assert np.array_equal(bf16_bits(summ), summ_o)
    for r in range(cfg.batch):
        res = oracle.coarse_to_fine_select(h["q"], h["w"], h["k"], h["s"], summ_o, h["ib"], r,
                                           topk_blocks=kb, n_recent_blocks=1, topk_tokens=kt)
        gb = [int(x) for x in bsel[r, :bn[r]].cpu()]
        gt = [int(x) for x in tsel[r, :tn[r]].cpu()]
        assert len(gb) == len(res["blocks"]) and len(gt) == kt
        if gb == res["blocks"]:
            full = np.full(cfg.context, -np.inf)
            for t, v in res["token_scores"].items():
                full[t] = v
            _check_topk(gt, full, sorted(res["token_scores"]), kt, f"tokens r{r}")
        _check_mla(inp, h, out, lse, r, gt, torch.bfloat16, sm, f"mla r{r}")
        say(f"  r{r}: blocks match {gb == res['blocks']}")


def test_indexer_fp8_codes_exact():
    """Token t carries fp8 code t in dim 0 (NaN codes replaced by 0); with
    q_0 = e_0, w_0 = 1 and q_1 = -e_0, w_1 = -1 its score is exactly the
    decoded code value: pins the fp8 widening on every e4m3fn code."""
    say("indexer fp8 codes")
    dev = _dev()
    P, H = 64, 16
    codes = np.arange(256, dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0
    keys = np.zeros((4, P, 128), dtype=np.uint8)
    keys.reshape(256, 128)[:, 0] = codes
    q = np.zeros((1, H, 128), dtype=np.float32)
    q[0, 0, 0], q[0, 1, 0] = 1.0, -1.0
    w = np.zeros((1, H), dtype=np.float32)
    w[0, 0], w[0, 1] = 1.0, -1.0
    kt = torch.tensor(keys, device=dev).view(torch.float8_e4m3fn)
    qt = torch.tensor(q, device=dev).to(torch.bfloat16)
    wt = torch.tensor(w, device=dev)
    st = torch.ones(4, P, device=dev)
    b = ls.PagedBatch(torch.tensor([0, 4], dtype=torch.int32, device=dev),
                      torch.arange(4, dtype=torch.int32, device=dev),
                      torch.tensor([256], dtype=torch.int32, device=dev), 4)
    sc = torch.zeros(1, ls.indexer_score_stride("tokens", 256), device=dev)
    ls.indexer_select(qt, wt, kt, P, b, granularity="tokens", topk=8, max_selected=8,
                      key_scales=st, scores_out=sc)
    torch.cuda.synchronize()
    want = oracle.numerics.fp8e4m3fn_to_f64(codes)
    got = sc[0, :256].cpu().numpy().astype(np.float64)
    assert np.array_equal(got, want), np.nonzero(got != want)[0][:10]


def test_indexer_block_mode_950k_coarse_shape():
    """The coarse pass of the 950K coarse-to-fine workload at full shape: 4
    requests x 15,200 blocks of 64 tokens, block-mean keys (bf16), 64 heads,
    top-256 blocks + the last block (the 1024-thread workgroup top-k).
    Every candidate's score against the oracle's float64 Eq. 6 over the
    block means; the selection exact outside the near-tie band."""
    say("indexer blocks at 4 x 15,200 blocks")
    dev = _dev()
    B, H, P, nb, kb = 4, 64, 64, 15200, 256
    g = torch.Generator().manual_seed(77)
    npg = B * nb
    summ = torch.randn(npg, 128, generator=g).to(torch.bfloat16).to(dev)
    q = torch.randn(B, H, 128, generator=g).to(torch.bfloat16).to(dev)
    w = (torch.randn(B, H, generator=g) / 8).to(dev)
    perm = torch.randperm(npg, generator=g).to(torch.int32).to(dev)
    lens = [nb * P - 40, nb * P, nb * P - 1, nb * P - 63]   # partial and complete last blocks
    b = ls.PagedBatch(torch.arange(0, npg + 1, nb, dtype=torch.int32, device=dev), perm,
                      torch.tensor(lens, dtype=torch.int32, device=dev), nb)
    sc = torch.full((B, nb), float("nan"), device=dev)
    sel, cnt = ls.indexer_select(q, w, summ, P, b, granularity="blocks", topk=kb, n_recent=1,
                                 max_selected=kb + 2, scores_out=sc)
    torch.cuda.synchronize()
    qb, wb, sb = bf16_bits(q), w.cpu().numpy(), bf16_bits(summ)
    bv = BatchView(np.arange(0, npg + 1, nb), perm.cpu().numpy(), np.array(lens), P)
    for r in range(B):
        s = oracle.indexer_block_scores(qb, wb, sb, bv, r)
        ncomp = bv.num_complete(r)
        nbr = bv.num_blocks(r)
        forced = set(oracle.method.forced_blocks(nbr, ncomp, 0, 1))
        cands = [j for j in range(ncomp) if j not in forced]
        got = sc[r, cands].double().cpu().numpy()
        mag = np.abs(np.maximum(oracle.bf16_to_f64(sb[bv.pages(r)[cands]]) @
                                oracle.bf16_to_f64(qb[r]).T, 0.0)) @ np.abs(wb[r].astype(np.float64))
        assert np.all(np.abs(got - s[cands]) <= 1e-5 * mag + 1e-6), f"scores r{r}"
        gsel = [int(x) for x in sel[r, :cnt[r]].cpu()]
        assert len(gsel) == kb + len(forced) and forced <= set(gsel)
        full = np.full(nbr, -np.inf)
        full[:ncomp] = s
        band = _check_topk(sorted(set(gsel) - forced), full, cands, kb, f"blocks r{r}")
        say(f"  r{r}: {len(gsel)} blocks, band {band}")
