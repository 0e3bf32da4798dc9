"""GPU parity of the approximate token top-k (Vortex, "Making it fast":
monotonic remap into buckets, early exit filling from the boundary bucket).

Bit-exact against the oracle where the fp32 scores are exact (integer keys,
queries and weights: every product and partial sum is an integer below
2^24), so both sides see the same buckets; with real-valued scores, the
certain winners are kept, nothing certainly below the boundary bucket is
taken, the count is exact, and the recall of the exact top-k is at least
97% (the figure the page reports for its approximation).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from oracle.method import BatchView, remap_bucket
from parity_util import say
from workloads import INDEXER_128K, bf16_bits, fp8_bits, make_indexer_inputs, reduced

pytestmark = pytest.mark.gpu

ls = pytest.importorskip("query_aware_sparse_ls_amd")


def _dev():
    assert torch.cuda.is_available()
    return torch.device("cuda:0")


def _inputs(lens, seed, integer=False):
    P = 64
    blocks = max(1, -(-max(lens) // P))
    cfg = reduced(INDEXER_128K, batch=len(lens), context=blocks * P, seed=seed)
    inp = make_indexer_inputs(cfg, device=_dev())
    inp.seq_lens.copy_(torch.tensor(lens, dtype=torch.int32))
    if integer:
        g = torch.Generator().manual_seed(seed)
        inp.q_idx.copy_(torch.randint(-1, 2, inp.q_idx.shape, generator=g).to(torch.bfloat16))
        inp.head_w.copy_(torch.randint(0, 3, inp.head_w.shape, generator=g).float())
        k = torch.randint(-3, 4, inp.idx_keys.shape, generator=g).float()
        inp.idx_keys.copy_(k.to(torch.float8_e4m3fn))
        inp.idx_scale.fill_(1.0)
    return inp


def _run(inp, k, approx, cand=None, cnt=None):
    P = inp.cfg.page_size
    nb = max(1, int((inp.seq_lens.max().item() + P - 1) // P))
    b = ls.PagedBatch(inp.idx_indptr, inp.idx_indices, inp.seq_lens, nb)
    sel, n = ls.indexer_select(inp.q_idx, inp.head_w, inp.idx_keys, P, b, granularity="tokens",
                               topk=k, max_selected=max(k, 1), key_scales=inp.idx_scale,
                               cand_blocks=cand, cand_counts=cnt, approx=approx)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), n.cpu().numpy()


def _host(inp):
    P = inp.cfg.page_size
    bv = BatchView(inp.idx_indptr.cpu().numpy(), inp.idx_indices.cpu().numpy(),
                   inp.seq_lens.cpu().numpy(), P)
    return (bf16_bits(inp.q_idx), inp.head_w.cpu().numpy(), fp8_bits(inp.idx_keys),
            inp.idx_scale.cpu().numpy(), bv)


@pytest.mark.parametrize("k", [1, 100, 2048, 5000])
def test_approx_topk_integer_scores_bit_exact(k):
    """Integer scores: many equal scores per bucket, so the boundary bucket is
    large and its fill order (ascending tokens) decides; ragged lengths."""
    lens = [9000, 4500, 63, 1]
    inp = _inputs(lens, seed=70 + k, integer=True)
    say(f"approx top-k, integer scores, k {k}")
    sel, n = _run(inp, k, 1)
    q, w, kb, ks, bv = _host(inp)
    for r, L in enumerate(lens):
        s = oracle.indexer_token_scores(q, w, kb, ks, bv, r)
        assert np.all(s == np.round(s)) and np.abs(s).max(initial=0) < 2 ** 24
        want = oracle.approx_select_tokens(s, k)
        assert sel[r, :n[r]].tolist() == want, (r, len(want), int(n[r]))
        assert (sel[r, n[r]:] == -1).all()


def test_approx_topk_integer_scores_with_block_candidates():
    lens = [6000, 3000]
    inp = _inputs(lens, seed=77, integer=True)
    cand = torch.tensor([[0, 3, 7, 20, 50, 93], [1, 2, 40, 46, -1, -1]], dtype=torch.int32,
                        device=_dev())
    cnt = torch.tensor([6, 4], dtype=torch.int32, device=_dev())
    sel, n = _run(inp, 150, 1, cand, cnt)
    q, w, kb, ks, bv = _host(inp)
    P = inp.cfg.page_size
    for r, L in enumerate(lens):
        blocks = cand[r, :int(cnt[r])].tolist()
        toks = oracle.tokens_of_blocks(blocks, P, L)
        s = oracle.indexer_token_scores(q, w, kb, ks, bv, r, tokens=toks)
        pick = oracle.approx_select_tokens(s, 150)
        assert sel[r, :n[r]].tolist() == sorted(int(toks[i]) for i in pick)


@pytest.mark.parametrize("seed", [78, 79])
def test_approx_topk_real_scores_properties_and_recall(seed):
    """Real-valued scores (the indexer workload's recipe, 128K and a ragged
    70,000-token request): the count is exact, every unit whose bucket is
    more than one above the boundary bucket is kept, nothing more than one
    bucket below it is taken (the kernel's fp32 scores may sit on the other
    side of a bucket edge from the oracle's), and the recall of the exact
    top-k is at least 97%."""
    lens = [131072, 70000]
    inp = _inputs(lens, seed=seed)
    k = 2048
    say(f"approx top-k, real scores, seed {seed}")
    sel, n = _run(inp, k, 1)
    ex, exn = _run(inp, k, 0)
    q, w, kb, ks, bv = _host(inp)
    for r, L in enumerate(lens):
        s = oracle.indexer_token_scores(q, w, kb, ks, bv, r)
        b = remap_bucket(s)
        kth = np.sort(b)[::-1][k - 1]
        got = set(sel[r, :n[r]].tolist())
        assert int(n[r]) == k and (sel[r, n[r]:] == -1).all()
        assert {i for i in range(L) if b[i] > kth + 1} <= got
        assert all(b[i] >= kth - 1 for i in got)
        exact = set(ex[r, :exn[r]].tolist())
        rec = len(got & exact) / k
        say(f"request {r}: recall of the approximate top-{k}: {rec:.4f}, "
            f"boundary bucket {int((b == kth).sum())} units")
        assert rec >= 0.97
