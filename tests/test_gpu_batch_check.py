"""GPU tests of the batch check (ls_check_batch) and of debug mode, in which
every call that takes a batch checks it first.

The expected reports are written out by hand from the batches below, which
are built to break one rule of the ls_batch contract each (the CSR page
table of the Vortex post's vTensor, "Why New Ideas Are Hard to Deploy"):
the kinds found, the number of violating requests, the first one, the count
of requests checked. The debug-mode call uses a negative length, which every
kernel reads as 0: its output must equal the same call with length 0.
"""

import math

import pytest
import torch

from parity_util import paged_batch, say
from workloads import LLAMA8B_32K_B16, make_block_topk_inputs, reduced

pytestmark = pytest.mark.gpu

ls = pytest.importorskip("query_aware_sparse_ls_amd")

P, NUM_PAGES, MAX_BLOCKS = 16, 20, 4

# (pages in the request's list, length, kinds expected)
REQUESTS = [
    ([1, 2, 3], 40, 0),                                            # valid
    ([4], -5, ls.LS_BATCH_NEGATIVE_LENGTH),
    ([5], 20, ls.LS_BATCH_LENGTH_BEYOND_PAGES),                     # 2 blocks, 1 page
    ([6, 7, 8, 9, 10], 80, ls.LS_BATCH_LENGTH_BEYOND_MAX_BLOCKS),   # 5 blocks > 4
    ([11, 20], 32, ls.LS_BATCH_PAGE_OUT_OF_RANGE),                  # page 20 of 20 is read
    ([12, 99], 16, 0),                                              # page 99 is never read
    ([13, -1, 14], 48, ls.LS_BATCH_PAGE_OUT_OF_RANGE),
    ([15, 16], 33, ls.LS_BATCH_LENGTH_BEYOND_PAGES),                # 3 blocks, 2 pages
    ([], 0, 0),                                                     # empty request
]


def _dev():
    assert torch.cuda.is_available()
    return torch.device("cuda:0")


def _batch(reqs, indptr=None):
    pages = [p for pg, _, _ in reqs for p in pg]
    if indptr is None:
        indptr = [0]
        for pg, _, _ in reqs:
            indptr.append(indptr[-1] + len(pg))
    t = lambda x: torch.tensor(x, dtype=torch.int32, device=_dev())
    return ls.PagedBatch(t(indptr), t(pages if pages else [0]), t([L for _, L, _ in reqs]),
                         MAX_BLOCKS)


def test_check_batch_each_kind_alone():
    say("batch check: one request per kind")
    for pg, L, kinds in REQUESTS:
        rep = ls.check_batch(_batch([(pg, L, kinds)]), P, NUM_PAGES).cpu().tolist()
        assert rep == [kinds, 1 if kinds else 0, 0 if kinds else -1, 1], (pg, L, rep)


def test_check_batch_whole_batch_and_bad_indptr():
    say("batch check: the whole batch, then a decreasing index pointer")
    rep = ls.check_batch(_batch(REQUESTS), P, NUM_PAGES).cpu().tolist()
    kinds = 0
    for _, _, k in REQUESTS:
        kinds |= k
    bad = [i for i, (_, _, k) in enumerate(REQUESTS) if k]
    assert rep == [kinds, len(bad), bad[0], len(REQUESTS)]
    # request 1's list ends before it starts: only that request is flagged
    # (its length 10 needs a block, which the empty list cannot hold)
    reqs = [([1, 2], 20, 0), ([3, 4], 10, 0), ([5], 16, 0)]
    rep = ls.check_batch(_batch(reqs, indptr=[0, 2, 1, 5]), P, NUM_PAGES).cpu().tolist()
    assert rep == [ls.LS_BATCH_BAD_INDPTR | ls.LS_BATCH_LENGTH_BEYOND_PAGES, 1, 1, 3]


def test_check_batch_clean_workload_and_empty_batch():
    cfg = reduced(LLAMA8B_32K_B16, batch=4, context=5000, page_table="pool",
                  pool_occupancy=0.5)
    say(f"batch check: a valid workload batch ({cfg.name}) and an empty one")
    inp = make_block_topk_inputs(cfg, device="cuda", seed=64)
    rep = ls.check_batch(paged_batch(inp), cfg.page_size, inp.k_pool.shape[0]).cpu().tolist()
    assert rep == [0, 0, -1, cfg.batch]
    e = torch.zeros(1, dtype=torch.int32, device=_dev())
    empty = ls.PagedBatch(e, e, e[:0], 1)
    assert ls.check_batch(empty, P, NUM_PAGES).cpu().tolist() == [0, 0, -1, 0]


def test_debug_mode_checks_every_call():
    """Debug mode on: two calls on a valid batch add nothing but their count;
    a call whose batch holds two negative lengths adds one violating call and
    two violating requests, and its output equals the call with length 0.
    Debug mode off: calls add nothing."""
    lens = [65541, 0, 1, 15, 16, 17, 8191, 8192, 8193, 65536, 40000, 33, 511 * 16 + 3,
            512 * 16, 512 * 16 + 1, 30000]
    lens = (lens * 2)[:32]
    cfg = reduced(LLAMA8B_32K_B16, batch=32, num_q_heads=32, num_kv_heads=8, head_dim=64,
                  context=max(lens))
    say(f"debug mode over dense calls: {cfg.name}")
    inp = make_block_topk_inputs(cfg, device="cuda", seed=61, seq_lens=lens)
    good = paged_batch(inp)
    neg = inp.seq_lens.clone()
    neg[torch.tensor([1, 17], device=neg.device)] = -7
    badb = ls.PagedBatch(good.page_indptr, good.page_indices, neg, good.max_blocks)
    sm = 1.0 / math.sqrt(cfg.head_dim)

    def call(b):
        out, _ = ls.sparse_attn_decode(inp.q, inp.k_pool, inp.v_pool, b, None, None,
                                       sm_scale=sm, out_dtype=torch.float32)
        torch.cuda.synchronize()
        return out

    was = ls.debug_enabled()
    try:
        ls.debug_enable(True)
        ls.debug_report()                      # start from zero
        ref = call(good)
        again = call(good)
        assert ls.debug_report() == (0, 0, 0, 2)
        got = call(badb)
        assert ls.debug_report() == (ls.LS_BATCH_NEGATIVE_LENGTH, 1, 2, 1)
        assert torch.equal(got, ref) and torch.equal(again, ref)
        ls.debug_enable(False)
        call(badb)
        assert ls.debug_report() == (0, 0, 0, 0)
    finally:
        ls.debug_enable(was)
