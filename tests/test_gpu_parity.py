"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Selections must equal the oracle's outside the near-tie band (1e-4 relative
to the k-th score); summaries bit-exact; attention outputs within 2e-2 (bf16)
or 1e-5 (fp32) of the oracle's attention over the GPU's own selection.
"""

import math

import numpy as np

import oracle
import pytest
import torch

from parity_util import (check_pair, complete_pages, paged_batch, poison_padding,
                         run_gpu_step, say, max_selected_for)
from oracle.method import topk_from_keep_ratio
from workloads import (LLAMA8B_32K_B16, TINY_4K, RAGGED_B64, make_block_topk_inputs, reduced,
                       bf16_bits)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import query_aware_sparse_ls_amd as ls
    say("libls:", ls.version(), ls._lib.LIB_PATH)


def _all_pairs(inp, **kw):
    res = kw.pop("res")
    bands = 0
    for r in range(inp.cfg.batch):
        for g in range(inp.cfg.num_kv_heads):
            bands += check_pair(inp, res, r, g, **kw)["band"]
    return bands


def _kw(inp, res, **over):
    cfg = inp.cfg
    kw = dict(res=res, topk=inp.topk, n_sink=cfg.n_sink, n_recent=cfg.n_recent,
              agg=cfg.group_agg, sm_scale=1.0 / math.sqrt(cfg.head_dim),
              out_dtype=torch.float32 if cfg.out_dtype == "fp32" else torch.bfloat16)
    kw.update(over)
    return kw


def test_tiny_4k_full_step():
    say("tiny 4K step: B1 Hq8 Hkv2 D64 L4096 top16+sink1+recent1 fp32 out")
    inp = make_block_topk_inputs(TINY_4K, device="cuda")
    res = run_gpu_step(inp)
    _all_pairs(inp, **_kw(inp, res))
    # the 8 hot blocks of each kv head must be among the selected
    for (r, g), hot in inp.hot_blocks.items():
        sel = set(res.selected[r, g, :int(res.counts[r, g])].tolist())
        assert set(hot) <= sel


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("agg", ["max", "mean"])
def test_tiny_4k_dtypes_and_aggregators(out_dtype, agg):
    say(f"tiny 4K: out {out_dtype} agg {agg}")
    inp = make_block_topk_inputs(TINY_4K, device="cuda", seed=7)
    res = run_gpu_step(inp, out_dtype=out_dtype, agg=agg)
    _all_pairs(inp, **_kw(inp, res, agg=agg, out_dtype=out_dtype))


def test_llama8b_shape_reduced_batch_context():
    cfg = reduced(LLAMA8B_32K_B16, batch=3, context=4096 + 5)
    say(f"8B shape reduced: {cfg}")
    inp = make_block_topk_inputs(cfg, device="cuda")
    res = run_gpu_step(inp)
    _all_pairs(inp, **_kw(inp, res))


def test_dense_k_all_matches_dense_oracle():
    cfg = reduced(LLAMA8B_32K_B16, batch=2, context=3000)
    say(f"dense k=all: {cfg}")
    inp = make_block_topk_inputs(cfg, device="cuda", seed=11)
    res = run_gpu_step(inp, dense=True, out_dtype=torch.float32)
    _all_pairs(inp, **_kw(inp, res, dense=True, out_dtype=torch.float32))


def test_topk_covering_everything_equals_dense():
    cfg = reduced(TINY_4K, context=700)
    say("top-k >= candidates: selection is every block and equals dense")
    inp = make_block_topk_inputs(cfg, device="cuda", seed=3)
    res = run_gpu_step(inp, topk=1000, out_dtype=torch.float32)
    dense = run_gpu_step(inp, dense=True, out_dtype=torch.float32)
    nb = -(-700 // 16)
    for g in range(cfg.num_kv_heads):
        assert res.selected[0, g, :int(res.counts[0, g])].tolist() == list(range(nb))
    # the dense call runs its own split-K kernels: equal up to rounding
    torch.testing.assert_close(res.out, dense.out, rtol=0, atol=1e-5)
    torch.testing.assert_close(res.lse, dense.lse, rtol=2e-6, atol=2e-5)
    _all_pairs(inp, **_kw(inp, dense, dense=True, out_dtype=torch.float32))


@pytest.mark.parametrize("L", [1, 15, 16, 17, 31, 33, 64, 200])
def test_short_and_ragged_edges(L):
    cfg = reduced(TINY_4K, context=L, n_hot=0)
    say(f"edge L={L}")
    inp = make_block_topk_inputs(cfg, device="cuda", seed=100 + L)
    for topk in (0, 1, 3):
        res = run_gpu_step(inp, topk=topk, n_sink=1, n_recent=1)
        _all_pairs(inp, **_kw(inp, res, topk=topk, n_sink=1, n_recent=1))
    res = run_gpu_step(inp, topk=2, n_sink=0, n_recent=0)
    _all_pairs(inp, **_kw(inp, res, topk=2, n_sink=0, n_recent=0))


def test_ragged_batch_pool_with_poisoned_unused_pages():
    cfg = reduced(RAGGED_B64, batch=6, ragged_range=(100, 6000), topk=8, keep_ratio=None,
                  pool_occupancy=0.7)
    say(f"ragged pool, NaN-poisoned unused pages: {cfg}")
    inp = make_block_topk_inputs(cfg, device="cuda", poison_unused=True)
    assert inp.unused_pages is not None and len(inp.unused_pages) > 0
    assert poison_padding(inp) > 0
    res = run_gpu_step(inp)
    assert torch.isfinite(res.out.float()).all()
    _all_pairs(inp, **_kw(inp, res))


@pytest.mark.parametrize("ratio", [1 / 64, 1 / 16, 1 / 4, 1.0])
def test_keep_ratio_budget(ratio):
    cfg = reduced(RAGGED_B64, batch=4, ragged_range=(300, 9000))
    say(f"keep ratio {ratio}")
    inp = make_block_topk_inputs(cfg, device="cuda", seed=21)
    res = run_gpu_step(inp, topk=-1, keep_ratio=ratio)
    P = cfg.page_size
    for r, L in enumerate(inp.seq_lens.tolist()):
        k = topk_from_keep_ratio(-(-L // P), L // P, ratio, cfg.n_sink, cfg.n_recent)
        for g in range(cfg.num_kv_heads):
            check_pair(inp, res, r, g, **{kk: v for kk, v in _kw(inp, res, topk=k).items()
                                           if kk != "res"})


@pytest.mark.parametrize("context", [1024, 8192])
def test_duplicate_summaries_tie_to_lowest_index(context):
    cfg = reduced(TINY_4K, context=context, n_hot=0)
    say(f"ties: identical pages, lowest block index wins (L={context})")
    inp = make_block_topk_inputs(cfg, device="cuda", seed=5)
    # make every page identical: every candidate ties exactly
    inp.k_pool[:] = inp.k_pool[0:1].clone()
    res = run_gpu_step(inp, topk=5, n_sink=1, n_recent=1)
    nb = context // 16
    for g in range(cfg.num_kv_heads):
        got = res.selected[0, g, :int(res.counts[0, g])].tolist()
        assert got == [0, 1, 2, 3, 4, 5, nb - 1], got


def test_page_permutation_invariance_and_determinism():
    cfg = reduced(LLAMA8B_32K_B16, batch=2, context=2048, page_table="contiguous")
    say("permutation invariance + bitwise determinism")
    inp = make_block_topk_inputs(cfg, device="cuda", seed=9)
    a = run_gpu_step(inp)
    b = run_gpu_step(inp)
    assert torch.equal(a.selected, b.selected) and torch.equal(a.out, b.out)
    assert torch.equal(a.lse, b.lse) and torch.equal(a.summaries, b.summaries)
    # move the pages to new physical slots
    n = inp.num_pages
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(1)).cuda()
    k2 = torch.empty_like(inp.k_pool); v2 = torch.empty_like(inp.v_pool)
    k2[perm] = inp.k_pool; v2[perm] = inp.v_pool
    inp2 = type(inp)(inp.cfg, inp.q, k2, v2, inp.page_indptr,
                     perm[inp.page_indices.long()].to(torch.int32), inp.seq_lens, inp.topk,
                     inp.hot_blocks)
    c = run_gpu_step(inp2)
    assert torch.equal(a.selected, c.selected) and torch.equal(a.out, c.out)


def test_llama8b_32k_b16_full_size_sampled():
    """The 8B / 32K / batch-16 step at full size; every selection and a sample
    of (request, kv head) outputs checked against the oracle."""
    cfg = LLAMA8B_32K_B16
    say(f"full size: {cfg}")
    inp = make_block_topk_inputs(cfg, device="cuda")
    res = run_gpu_step(inp)
    rng = np.random.default_rng(0)
    pairs = {(0, 0), (15, 7)} | {(int(rng.integers(16)), int(rng.integers(8))) for _ in range(6)}
    bands = 0
    for r, g in sorted(pairs):
        bands += check_pair(inp, res, r, g, **{k: v for k, v in _kw(inp, res).items()
                                               if k != "res"})["band"]
    # every (r, g) selection against the oracle's ranking of the GPU summaries
    # (those are bit-exact wherever checked above)
    from oracle.method import BatchView
    from parity_util import check_selection
    summ = bf16_bits(res.summaries)
    bv = BatchView(inp.page_indptr.cpu().numpy(), inp.page_indices.cpu().numpy(),
                   inp.seq_lens.cpu().numpy(), cfg.page_size)
    q = bf16_bits(inp.q)
    hot_hit = hot_all = 0
    for r in range(cfg.batch):
        for g in range(cfg.num_kv_heads):
            s = oracle.block_scores(q, summ, bv, r, g, num_kv_heads=cfg.num_kv_heads, agg="max")
            sel = res.selected[r, g, :int(res.counts[r, g])].tolist()
            bands += check_selection(sel, s, 2048, 2048, cfg.topk, cfg.n_sink, cfg.n_recent)["band"]
            hot = inp.hot_blocks[(r, g)]
            hot_hit += len(set(hot) & set(sel))
            hot_all += len(hot)
    assert (res.counts == 67).all()
    # the +2 sigma hot blocks dominate the selection (not all: a hot block can
    # still rank below the 64th score)
    assert hot_hit >= 0.95 * hot_all, (hot_hit, hot_all)
    say(f"near-tie band blocks: {bands}; hot blocks selected {hot_hit}/{hot_all}")


def test_ragged_many_pairs_long_requests_keep_ratio():
    """The batch-64 ragged sweep's shape class: 264 (request, kv head) pairs,
    lengths log-uniform in [2K, 128K] (requests of up to 8192 blocks), keep
    ratio 1/16 -- the many-workgroups route with 8192-block ranking rows.
    Sampled pairs (the shortest, the longest, and two in between) against the
    oracle; the fused step equals the separate calls bit for bit."""
    from parity_util import run_gpu_fused
    cfg = reduced(RAGGED_B64, batch=33)
    say(f"ragged {cfg.batch} requests, 2K-128K, keep 1/16")
    inp = make_block_topk_inputs(cfg, device="cuda", seed=24)   # longest: 112,317 tokens
    lens = inp.seq_lens.tolist()
    assert max(lens) > 16 * 4096, "a request of more than 4096 blocks"
    res = run_gpu_step(inp, topk=-1, keep_ratio=cfg.keep_ratio)
    fus = run_gpu_fused(inp, summaries=res.summaries, topk=-1, keep_ratio=cfg.keep_ratio)
    assert torch.equal(res.counts, fus.counts)
    assert torch.equal(res.out, fus.out) and torch.equal(res.lse, fus.lse)
    P = cfg.page_size
    order = np.argsort(lens)
    for r in (int(order[0]), int(order[-1]), int(order[len(lens) // 2]), int(order[-2])):
        L = lens[r]
        k = topk_from_keep_ratio(-(-L // P), L // P, cfg.keep_ratio, cfg.n_sink, cfg.n_recent)
        for g in (0, 7):
            say(f"  r{r} (L={L}) g{g}")
            check_pair(inp, res, r, g, **{kk: v for kk, v in _kw(inp, res, topk=k).items()
                                           if kk != "res"})


@pytest.mark.parametrize("keep", [1.0 / 64, 1.0 / 4])
def test_ragged_b64_full_size_keep_ratios(keep):
    """The batch-64 ragged sweep at full size (512 pairs, lengths log-uniform
    in [2K, 128K], shared pool at 70% occupancy): the planned route. Fused
    step equal to the separate calls; sampled pairs (the shortest, the
    longest, two in between) against the oracle."""
    from parity_util import run_gpu_fused
    cfg = RAGGED_B64
    say(f"ragged B64 full size, keep {keep}")
    inp = make_block_topk_inputs(cfg, device="cuda", seed=cfg.seed)
    lens = inp.seq_lens.tolist()
    assert max(lens) > 16 * 4096
    res = run_gpu_step(inp, topk=-1, keep_ratio=keep)
    fus = run_gpu_fused(inp, summaries=res.summaries, topk=-1, keep_ratio=keep)
    assert torch.equal(res.counts, fus.counts)
    assert torch.equal(res.out, fus.out) and torch.equal(res.lse, fus.lse)
    P = cfg.page_size
    order = np.argsort(lens)
    for r in (int(order[0]), int(order[-1]), int(order[len(lens) // 3]), int(order[-5])):
        L = lens[r]
        k = topk_from_keep_ratio(-(-L // P), L // P, keep, cfg.n_sink, cfg.n_recent)
        for g in (0, 5):
            say(f"  r{r} (L={L}) g{g}")
            check_pair(inp, res, r, g, **{kk: v for kk, v in _kw(inp, res, topk=k).items()
                                           if kk != "res"})
