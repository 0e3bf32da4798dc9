"""GPU parity of Quest bound scoring (score_mode "bounds"): the bounds builder
against the oracle's element-wise max/min, and the selection + attention
built on the bounds (separate calls and the fused step, which must agree bit
for bit) against the oracle's bound scores, top-k and attention.

Bounds: exact (values; the sign of a zero bound is not specified). Scores
within 1e-5 relative of the fp64 oracle; selections exact outside the near-tie
band; outputs within 2e-2 (bf16) or 1e-5 (fp32).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle.method import forced_blocks
from parity_util import (GpuStep, build_summaries, check_pair, run_gpu_fused,
                         run_gpu_step, say)
from workloads import LLAMA8B_32K_B16, TINY_4K, bf16_bits, make_block_topk_inputs, reduced

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import query_aware_sparse_ls_amd as ls
    say("libls:", ls.version(), ls._lib.LIB_PATH)


def _kw(inp, **over):
    cfg = inp.cfg
    kw = dict(topk=inp.topk, n_sink=cfg.n_sink, n_recent=cfg.n_recent, agg=cfg.group_agg,
              sm_scale=1.0 / math.sqrt(cfg.head_dim),
              out_dtype=torch.float32 if cfg.out_dtype == "fp32" else torch.bfloat16,
              score_mode="bounds")
    kw.update(over)
    return kw


def _pairs(cfg, n, seed=0):
    rng = np.random.default_rng(seed)
    allp = [(r, g) for r in range(cfg.batch) for g in range(cfg.num_kv_heads)]
    pick = {allp[0], allp[-1]}
    for i in rng.permutation(len(allp))[:n]:
        pick.add(allp[int(i)])
    return sorted(pick)


def _same(a: GpuStep, b: GpuStep):
    assert torch.equal(a.counts, b.counts)
    for r in range(a.counts.shape[0]):
        for g in range(a.counts.shape[1]):
            n = int(a.counts[r, g])
            assert torch.equal(a.selected[r, g, :n], b.selected[r, g, :n])
    assert torch.equal(a.out, b.out)
    assert torch.equal(a.lse, b.lse)


def _values_equal(a_bits: np.ndarray, b_bits: np.ndarray) -> bool:
    return np.array_equal(oracle.bf16_to_f64(a_bits), oracle.bf16_to_f64(b_bits))


@pytest.mark.parametrize("D,P", [(128, 16), (64, 16), (128, 32), (64, 64)])
def test_bounds_match_oracle_and_leave_other_pages(D, P):
    """Bounds of a listed subset of pages (in a shuffled order, one listed
    twice) equal the oracle's max/min; unlisted pages keep their contents.
    Keys include zeros of both signs and whole constant columns."""
    import query_aware_sparse_ls_amd as ls
    H, pages = 8, 300
    g = torch.Generator().manual_seed(D * 1000 + P)
    k = (torch.randn(pages, H, P, D, generator=g) * 3).to(torch.bfloat16)
    k[5, :, :, :4] = 0.0
    k[5, :, ::2, 4:8] = -0.0
    k[9, 2] = k[9, 2, 0]                     # every token of the block equal
    k[11, :, 3, 7] = 65504.0
    ids = torch.randperm(pages, generator=g)[:200].to(torch.int32)
    ids = torch.cat([ids, ids[:1]])
    say(f"bounds builder: D {D}, P {P}, {ids.numel()} pages listed")
    sentinel = torch.full((pages, H, 2, D), 7.0, dtype=torch.bfloat16)
    out = sentinel.cuda()
    ls.build_block_bounds(k.cuda(), ids.cuda(), out)
    torch.cuda.synchronize()
    got = bf16_bits(out.cpu())
    want = oracle.block_bounds(bf16_bits(k), ids.numpy())
    assert _values_equal(got[ids.numpy()], want)
    unlisted = np.setdiff1d(np.arange(pages), ids.numpy())
    assert np.array_equal(got[unlisted], bf16_bits(sentinel)[unlisted])


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("agg", ["max", "mean"])
def test_quest_many_pairs_d128(agg, out_dtype):
    """128 pairs of ragged requests (one fused launch): separate calls and the
    fused step agree bit for bit, and both match the oracle."""
    lens = [9000, 1, 17, 33, 4096, 4111, 100, 31, 8191, 2048, 15000, 16, 700, 3000, 5555, 48]
    cfg = reduced(LLAMA8B_32K_B16, context=max(lens), group_agg=agg,
                  out_dtype="fp32" if out_dtype == torch.float32 else "bf16")
    say(f"quest, 128 pairs: agg {agg}, out {out_dtype}")
    inp = make_block_topk_inputs(cfg, device="cuda", seed=91, seq_lens=lens)
    sep = run_gpu_step(inp, score_mode="bounds")
    fus = run_gpu_fused(inp, summaries=sep.summaries, score_mode="bounds")
    _same(sep, fus)
    for r, g in _pairs(cfg, 10, seed=1) + [(1, 0), (2, 5), (11, 3)]:
        check_pair(inp, sep, r, g, **_kw(inp))


def test_quest_many_pairs_d64():
    """Head dim 64, 64 pairs, fp32 output."""
    cfg = reduced(TINY_4K, batch=32, context=6000, n_hot=10)
    say(f"quest, d64: {cfg.name}")
    inp = make_block_topk_inputs(cfg, device="cuda", seed=92)
    sep = run_gpu_step(inp, score_mode="bounds")
    fus = run_gpu_fused(inp, summaries=sep.summaries, score_mode="bounds")
    _same(sep, fus)
    for r, g in _pairs(cfg, 8, seed=2):
        check_pair(inp, sep, r, g, **_kw(inp))


@pytest.mark.parametrize("name,cfg", [
    ("2 requests, 16 pairs", reduced(LLAMA8B_32K_B16, batch=2, context=20000)),
    ("long requests, 128 pairs", reduced(LLAMA8B_32K_B16, batch=16, context=100000)),
])
def test_quest_split_launch_forms(name, cfg):
    """Batches the fused kernel does not take in bounds mode (few pairs; or
    requests over 4096 blocks in at most 256 pairs) run bounds selection
    then attention: same results as the separate calls, oracle parity."""
    say(f"quest, separate launches inside the step: {name}")
    inp = make_block_topk_inputs(cfg, device="cuda", seed=93)
    sep = run_gpu_step(inp, score_mode="bounds")
    fus = run_gpu_fused(inp, summaries=sep.summaries, score_mode="bounds")
    _same(sep, fus)
    for r, g in _pairs(cfg, 4, seed=3):
        check_pair(inp, sep, r, g, **_kw(inp))


@pytest.mark.parametrize("batch", [16, 2])   # one launch (128 pairs) / separate launches
def test_quest_step_refreshes_bounds_of_pages_that_filled(batch):
    """Every request's last page just filled: the step rebuilds those pages'
    bounds itself (rows start as NaN) and gives the same bounds, selections
    and outputs, bit for bit, as building them first."""
    cfg = reduced(LLAMA8B_32K_B16, batch=batch, context=4096)
    say(f"quest step with bounds refresh, batch {batch}")
    inp = make_block_topk_inputs(cfg, device="cuda", seed=94)
    P = cfg.page_size
    indptr = inp.page_indptr.cpu().tolist()
    idx = inp.page_indices.cpu()
    new = torch.tensor([int(idx[indptr[r] + cfg.context // P - 1]) for r in range(batch)],
                       dtype=torch.int32, device="cuda")
    full = build_summaries(inp, "bounds")
    stale = full.clone()
    stale[new.long()] = float("nan")
    a = run_gpu_fused(inp, summaries=stale, new_pages=new, score_mode="bounds")
    b = run_gpu_fused(inp, summaries=full, score_mode="bounds")
    assert torch.equal(stale.view(torch.int16), full.view(torch.int16))
    _same(a, b)
    want = oracle.block_bounds(bf16_bits(inp.k_pool), new.cpu().numpy())
    assert _values_equal(bf16_bits(stale)[new.cpu().numpy()], want)


def test_quest_full_size_llama8b_32k_b16():
    """The bench's bounds step (16 requests x 32K, 128 pairs, top-64 + 1 sink
    + 2 recent): sampled pairs against the oracle; two calls bit-identical."""
    cfg = LLAMA8B_32K_B16
    say(f"quest at full size: {cfg.name}")
    inp = make_block_topk_inputs(cfg, device="cuda")
    bounds = build_summaries(inp, "bounds")
    a = run_gpu_fused(inp, summaries=bounds, score_mode="bounds")
    b = run_gpu_fused(inp, summaries=bounds, score_mode="bounds")
    _same(a, b)
    sep = run_gpu_step(inp, score_mode="bounds")
    _same(sep, a)
    for r, g in [(0, 0), (7, 3), (15, 7)]:
        check_pair(inp, sep, r, g, **_kw(inp))


def test_quest_bounds_never_below_the_best_token_score():
    """Property at any size: for every sampled candidate block, the GPU's
    bound score (max over the group) is at least the largest exact q . k of
    the block's tokens (up to fp32 rounding of the sums)."""
    cfg = reduced(LLAMA8B_32K_B16, batch=4, context=3000)
    inp = make_block_topk_inputs(cfg, device="cuda", seed=95)
    res = run_gpu_step(inp, score_mode="bounds", topk=8)
    P, G = cfg.page_size, cfg.group
    for r, g in _pairs(cfg, 6, seed=4):
        L = int(inp.seq_lens[r])
        nc = L // P
        p0 = int(inp.page_indptr[r])
        pages = inp.page_indices[p0:p0 + nc].long()
        k = inp.k_pool[pages, g].float()                       # [nc][P][D]
        q = inp.q[r, g * G:(g + 1) * G].float()                # [G][D]
        best = torch.matmul(k, q.t().contiguous()).amax(dim=(1, 2))   # [nc]
        forced = set(forced_blocks(-(-L // P), nc, cfg.n_sink, cfg.n_recent))
        cands = [j for j in range(nc) if j not in forced]
        s = res.scores[r, g, cands]
        slack = 1e-5 * (1.0 + best[cands].abs())
        assert bool((s >= best[cands] - slack).all())
