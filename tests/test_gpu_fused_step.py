"""The whole decode step in one call (ls_sparse_decode_step): identical to
the separate calls, correct against the oracle, reusable workspace, and
replayable from a HIP graph."""

import math

import numpy as np
import pytest
import torch

from parity_util import check_pair, run_gpu_fused, run_gpu_step, say
from workloads import LLAMA8B_32K_B16, TINY_4K, RAGGED_B64, make_block_topk_inputs, reduced

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _kw(inp, **over):
    cfg = inp.cfg
    kw = dict(topk=inp.topk, n_sink=cfg.n_sink, n_recent=cfg.n_recent, agg=cfg.group_agg,
              sm_scale=1.0 / math.sqrt(cfg.head_dim),
              out_dtype=torch.float32 if cfg.out_dtype == "fp32" else torch.bfloat16)
    kw.update(over)
    return kw


def _same(a, b):
    assert torch.equal(a.counts, b.counts)
    for r in range(a.counts.shape[0]):
        for g in range(a.counts.shape[1]):
            n = int(a.counts[r, g])
            assert torch.equal(a.selected[r, g, :n], b.selected[r, g, :n])
    assert torch.equal(a.out, b.out)
    assert torch.equal(a.lse, b.lse)


@pytest.mark.parametrize("cfg", [
    TINY_4K,
    reduced(LLAMA8B_32K_B16, batch=3, context=4096 + 5),
    reduced(LLAMA8B_32K_B16, batch=11, context=1000),
    reduced(RAGGED_B64, batch=9, ragged_range=(40, 5000), topk=8, keep_ratio=None),
    # 40 pairs: many workgroups per pair, the pair's last score chunk has candidates
    reduced(LLAMA8B_32K_B16, batch=5, context=2500),
    # 24 pairs of up to 5000 blocks: the 8192-block ranking
    reduced(RAGGED_B64, batch=3, ragged_range=(20000, 80000), topk=40, keep_ratio=None),
    # 72 pairs, the longest over 4096 blocks: the planned route (scoring and
    # attention cut into equal ranges across pairs)
    reduced(RAGGED_B64, batch=9, ragged_range=(17, 80000), topk=40, keep_ratio=None),
], ids=["tiny", "8b_b3", "8b_b11", "ragged_b9", "8b_b5_2500", "ragged_b3_long", "planned_b9"])
def test_fused_equals_separate_and_oracle(cfg):
    say(f"fused step vs separate calls and oracle: {cfg.name}")
    lens = None
    if cfg.batch == 9 and cfg.ragged_range == (17, 80000):
        # an empty request, one of a partial page, short and long ones
        lens = [80000, 2000, 35000, 65600, 17, 4100, 70001, 0, 50000]
    inp = make_block_topk_inputs(cfg, device="cuda", seed=31, seq_lens=lens)
    sep = run_gpu_step(inp)
    fus = run_gpu_fused(inp, summaries=sep.summaries)
    _same(sep, fus)
    for r in range(cfg.batch):
        for g in range(cfg.num_kv_heads):
            check_pair(inp, fus, r, g, **_kw(inp))


def test_fused_workspace_reuse_across_calls():
    say("fused step: one workspace, three different steps")
    import query_aware_sparse_ls_amd as ls
    cfg = reduced(LLAMA8B_32K_B16, batch=4, context=3000)
    ws = None
    for seed in (1, 2, 3):
        inp = make_block_topk_inputs(cfg, device="cuda", seed=seed)
        if ws is None:
            B, Hq, D = inp.q.shape
            ws = ls.sparse_decode_step_workspace(B, Hq, cfg.num_kv_heads, D, inp.max_blocks(),
                                                 inp.topk + 4, "cuda")
        sep = run_gpu_step(inp)
        fus = run_gpu_fused(inp, summaries=sep.summaries, workspace=ws)
        _same(sep, fus)
        # every hand-off word and the error word are back at zero
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(ws)) == 0


@pytest.mark.parametrize("batch,context", [
    (5, 2500),     # 40 pairs: many workgroups per pair
    (16, 2500),    # 128 pairs: one workgroup per pair
    (8, 70000),    # 64 pairs of 4375 blocks: the planned route
])
def test_workspace_left_zero_by_every_call(batch, context):
    """Selection, attention and step calls each leave their workspace zero
    (hand-off words reset by their readers, no wait gave up), also when one
    workspace serves all three in turn."""
    import query_aware_sparse_ls_amd as ls
    from parity_util import paged_batch
    cfg = reduced(LLAMA8B_32K_B16, batch=batch, context=context)
    inp = make_block_topk_inputs(cfg, device="cuda", seed=9)
    B, Hq, D = inp.q.shape
    Hkv = cfg.num_kv_heads
    batch = paged_batch(inp)
    maxsel = inp.topk + cfg.n_sink + cfg.n_recent + 1
    n = max(ls.score_select_workspace_size(B, Hkv, batch.max_blocks),
            ls.sparse_attn_decode_workspace_size(B, Hq, D, maxsel, batch.max_blocks),
            ls.sparse_decode_step_workspace(B, Hq, Hkv, D, batch.max_blocks, maxsel,
                                            "cuda").numel())
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    ref = run_gpu_step(inp)
    for it in range(3):
        sel, cnt = ls.score_select(inp.q, ref.summaries, cfg.page_size, batch, topk=inp.topk,
                                   n_sink=cfg.n_sink, n_recent=cfg.n_recent,
                                   max_selected=maxsel, workspace=ws)
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(ws)) == 0, f"select {it}"
        assert torch.equal(cnt, ref.counts)
        out, _ = ls.sparse_attn_decode(inp.q, inp.k_pool, inp.v_pool, batch, sel, cnt,
                                       sm_scale=1.0 / math.sqrt(D), workspace=ws)
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(ws)) == 0, f"attention {it}"
        out2, _, _, cnt2 = ls.sparse_decode_step(inp.q, ref.summaries, inp.k_pool, inp.v_pool,
                                                 batch, topk=inp.topk, n_sink=cfg.n_sink,
                                                 n_recent=cfg.n_recent, max_selected=maxsel,
                                                 sm_scale=1.0 / math.sqrt(D), workspace=ws)
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(ws)) == 0, f"step {it}"
        assert torch.equal(out, out2) and torch.equal(cnt2, ref.counts)


@pytest.mark.parametrize("batch,context", [(4, 5000), (8, 70000)])   # flow; planned (3 launches)
def test_fused_step_hip_graph_replay(batch, context):
    say(f"fused step captured in a HIP graph, replayed with eager work in between: "
        f"{batch} x {context}")
    import query_aware_sparse_ls_amd as ls
    cfg = reduced(LLAMA8B_32K_B16, batch=batch, context=context)
    inp = make_block_topk_inputs(cfg, device="cuda", seed=4)
    eager = run_gpu_step(inp)
    B, Hq, D = inp.q.shape
    batch = ls.PagedBatch(inp.page_indptr, inp.page_indices, inp.seq_lens, inp.max_blocks())
    maxsel = inp.topk + cfg.n_sink + cfg.n_recent + 1
    ws = ls.sparse_decode_step_workspace(B, Hq, cfg.num_kv_heads, D, batch.max_blocks, maxsel,
                                         "cuda")
    sel = torch.empty(B, cfg.num_kv_heads, maxsel, dtype=torch.int32, device="cuda")
    cnt = torch.empty(B, cfg.num_kv_heads, dtype=torch.int32, device="cuda")
    out = torch.empty(B, Hq, D, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, Hq, dtype=torch.float32, device="cuda")

    def step():
        ls.sparse_decode_step(inp.q, eager.summaries, inp.k_pool, inp.v_pool, batch,
                              topk=inp.topk, n_sink=cfg.n_sink, n_recent=cfg.n_recent,
                              max_selected=maxsel, sm_scale=1.0 / math.sqrt(D), selected=sel,
                              selected_count=cnt, out=out, lse=lse, workspace=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(5):
        out.zero_(); lse.zero_(); sel.fill_(-7); cnt.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager.out), f"replay {i}"
        assert torch.equal(lse, eager.lse)
        assert torch.equal(cnt, eager.counts)
        _ = run_gpu_step(inp)            # unrelated eager work between replays


def test_fused_full_size_llama8b_32k_b16():
    cfg = LLAMA8B_32K_B16
    say(f"fused step at full size: {cfg.name}")
    inp = make_block_topk_inputs(cfg, device="cuda")
    sep = run_gpu_step(inp)
    fus = run_gpu_fused(inp, summaries=sep.summaries)
    _same(sep, fus)
    for r, g in [(0, 0), (7, 3), (15, 7)]:
        check_pair(inp, fus, r, g, **_kw(inp))


@pytest.mark.parametrize("batch", [16, 2])   # 128 and 16 (request, kv head) pairs
def test_step_refreshes_pages_that_filled(batch):
    """Every request's last page just filled: the step rebuilds those pages'
    summaries itself (rows start as NaN) and gives the same summaries,
    selections and outputs, bit for bit, as building them first."""
    import query_aware_sparse_ls_amd as ls
    from oracle import block_summaries
    from parity_util import complete_pages
    from workloads import bf16_bits
    cfg = reduced(LLAMA8B_32K_B16, batch=batch, context=4096)
    say(f"step with summary refresh, batch {batch}")
    inp = make_block_topk_inputs(cfg, device="cuda", seed=31)
    P, Hkv, D = cfg.page_size, cfg.num_kv_heads, cfg.head_dim
    indptr = inp.page_indptr.cpu().tolist()
    idx = inp.page_indices.cpu()
    new = torch.tensor([int(idx[indptr[r] + cfg.context // P - 1]) for r in range(batch)],
                       dtype=torch.int32, device="cuda")
    full = torch.zeros(inp.num_pages, Hkv, D, dtype=torch.bfloat16, device="cuda")
    ls.build_block_summaries(inp.k_pool, complete_pages(inp).cuda(), full)
    stale = full.clone()
    stale[new.long()] = float("nan")
    a = run_gpu_fused(inp, summaries=stale, new_pages=new)
    b = run_gpu_fused(inp, summaries=full)
    assert torch.equal(stale.view(torch.int16), full.view(torch.int16))
    _same(a, b)
    want = block_summaries(bf16_bits(inp.k_pool), new.cpu().numpy())
    assert np.array_equal(bf16_bits(stale)[new.cpu().numpy()], want)
