"""Hand-offs between the workgroups of one launch (block scores, walk
entries, split states, token lists and bitmaps): every route that passes data
from one workgroup to another inside a launch gives the same bits with a
workspace zero-filled by a separate kernel right before the call as with a
reused one. Row lengths are not multiples of 32 words, so the rows of
neighbouring pairs share cache lines."""

import math

import pytest
import torch

from parity_util import paged_batch, run_gpu_fused, run_gpu_step, say
from workloads import (INDEXER_128K, LLAMA8B_32K_B16, RAGGED_B64, make_block_topk_inputs,
                       make_indexer_inputs, reduced)

pytestmark = pytest.mark.gpu

CALLS = 12


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _fresh(nbytes):
    # zero-filled by a fill kernel, as a caller's new workspace would be
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device="cuda")


def _same_step(a, b, what):
    assert torch.equal(a.counts, b.counts), what
    for r in range(a.counts.shape[0]):
        for g in range(a.counts.shape[1]):
            n = int(a.counts[r, g])
            assert torch.equal(a.selected[r, g, :n], b.selected[r, g, :n]), (what, r, g)
    assert torch.equal(a.out, b.out), what
    assert torch.equal(a.lse, b.lse), what


@pytest.mark.parametrize("cfg", [
    # 40 pairs of 157 blocks: the many-workgroups route (score chunks, ranker,
    # attention items, merger)
    reduced(LLAMA8B_32K_B16, batch=5, context=2500),
    # 72 pairs, the longest over 4096 blocks: the planned route (pairs cut by
    # range ends merged by their last workgroup)
    reduced(RAGGED_B64, batch=9, ragged_range=(17, 80000), topk=40, keep_ratio=None),
], ids=["flow_b5_2500", "planned_b9"])
def test_step_with_fresh_workspaces(cfg):
    import query_aware_sparse_ls_amd as ls
    say(f"step, a fresh zero-filled workspace per call: {cfg.name}")
    lens = None
    if cfg.batch == 9:
        lens = [80000, 2000, 35000, 65600, 17, 4100, 70001, 0, 50000]
    inp = make_block_topk_inputs(cfg, device="cuda", seed=17, seq_lens=lens)
    ref = run_gpu_step(inp)
    B, Hq, D = inp.q.shape
    Hkv = cfg.num_kv_heads
    maxsel = inp.topk + cfg.n_sink + cfg.n_recent + 1
    nbytes = ls.sparse_decode_step_workspace(B, Hq, Hkv, D, inp.max_blocks(), maxsel,
                                             "cuda").numel()
    for it in range(CALLS):
        got = run_gpu_fused(inp, summaries=ref.summaries, workspace=_fresh(nbytes))
        _same_step(ref, got, f"call {it}")


def test_separate_calls_with_fresh_workspaces():
    """ls_score_select and ls_sparse_attn_decode on the many-workgroups route
    (fewer than 64 pairs), each with a new zero-filled workspace."""
    import query_aware_sparse_ls_amd as ls
    cfg = reduced(LLAMA8B_32K_B16, batch=5, context=2500)
    say(f"separate calls, a fresh zero-filled workspace per call: {cfg.name}")
    inp = make_block_topk_inputs(cfg, device="cuda", seed=23)
    ref = run_gpu_step(inp)
    batch = paged_batch(inp)
    B, Hq, D = inp.q.shape
    Hkv = cfg.num_kv_heads
    maxsel = inp.topk + cfg.n_sink + cfg.n_recent + 1
    nsel = ls.score_select_workspace_size(B, Hkv, batch.max_blocks)
    natt = ls.sparse_attn_decode_workspace_size(B, Hq, D, maxsel, batch.max_blocks)
    for it in range(CALLS):
        sel, cnt = ls.score_select(inp.q, ref.summaries, cfg.page_size, batch, topk=inp.topk,
                                   n_sink=cfg.n_sink, n_recent=cfg.n_recent,
                                   max_selected=maxsel, workspace=_fresh(nsel))
        out, _ = ls.sparse_attn_decode(inp.q, inp.k_pool, inp.v_pool, batch, ref.selected,
                                       ref.counts, sm_scale=1.0 / math.sqrt(D),
                                       out_dtype=ref.out.dtype, workspace=_fresh(natt))
        torch.cuda.synchronize()
        assert torch.equal(cnt, ref.counts), f"call {it}"
        for r in range(B):
            for g in range(Hkv):
                n = int(ref.counts[r, g])
                assert torch.equal(sel[r, g, :n], ref.selected[r, g, :n]), (it, r, g)
        assert torch.equal(out, ref.out), f"call {it}"


@pytest.mark.parametrize("lens,topk", [((5000, 3001), 256), ((5120, 2500), 2048)])
def test_indexer_token_topk_with_fresh_workspaces(lens, topk):
    """The token top-k's finishing workgroup reads the boundary digit's listed
    units and the bitmap that the other workgroups handed over."""
    import query_aware_sparse_ls_amd as ls
    say(f"indexer token top-k, a fresh zero-filled workspace per call: lens={lens} topk={topk}")
    P = 64
    cfg = reduced(INDEXER_128K, batch=len(lens), context=80 * P, page_size=P, seed=7)
    inp = make_indexer_inputs(cfg, device="cuda")
    inp.seq_lens.copy_(torch.tensor(list(lens), dtype=torch.int32))
    nb = max(1, (max(lens) + P - 1) // P)
    b = ls.PagedBatch(inp.idx_indptr, inp.idx_indices, inp.seq_lens, nb)
    units = b.max_blocks * P
    nbytes = ls.indexer_select_workspace_size(cfg.batch, "tokens", units)

    def run(ws):
        sel, n = ls.indexer_select(inp.q_idx, inp.head_w, inp.idx_keys, P, b,
                                   granularity="tokens", topk=topk, max_selected=topk + 3,
                                   key_scales=inp.idx_scale, workspace=ws)
        torch.cuda.synchronize()
        return sel, n

    ref_sel, ref_n = run(_fresh(nbytes))
    reused = _fresh(nbytes)
    for it in range(CALLS):
        sel, n = run(_fresh(nbytes) if it % 2 == 0 else reused)
        assert torch.equal(n, ref_n), f"call {it}"
        assert torch.equal(sel, ref_sel), f"call {it}"
