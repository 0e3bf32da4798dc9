"""Helpers for GPU-vs-oracle parity tests (imported by tests only).

The HIP path runs through the C ABI (via the thin binding); the oracle gets
the same input bits, copied to the host, and recomputes everything itself.
"""

from __future__ import annotations

import math
import sys
from dataclasses import dataclass
from typing import Dict, List, Tuple

import numpy as np
import torch

import oracle
from oracle.method import BatchView, forced_blocks
from workloads import BlockTopKInputs, bf16_bits

BF16_ATOL = 2e-2
FP32_ATOL = 1e-5
TIE_REL = 1e-4
TIE_ABS_OF_MAX = 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@dataclass
class GpuStep:
    summaries: torch.Tensor
    scores: torch.Tensor
    selected: torch.Tensor
    counts: torch.Tensor
    out: torch.Tensor
    lse: torch.Tensor


def complete_pages(inp: BlockTopKInputs) -> torch.Tensor:
    """Physical ids of every complete page of every request (host-side list)."""
    P = inp.cfg.page_size
    indptr = inp.page_indptr.cpu().tolist()
    idx = inp.page_indices.cpu()
    ids = []
    for r, L in enumerate(inp.seq_lens.cpu().tolist()):
        ids.append(idx[indptr[r]:indptr[r] + L // P])
    return torch.cat(ids).to(torch.int32) if ids else torch.zeros(0, dtype=torch.int32)


def paged_batch(inp: BlockTopKInputs):
    import query_aware_sparse_ls_amd as ls
    return ls.PagedBatch(inp.page_indptr, inp.page_indices, inp.seq_lens, inp.max_blocks())


def max_selected_for(topk, n_sink, n_recent, max_blocks, keep_ratio=None):
    if topk >= 0:
        return min(max_blocks, topk + n_sink + n_recent + 1)
    by_ratio = math.ceil(float(np.float32(keep_ratio)) * max_blocks) + 1
    return min(max_blocks, max(n_sink + n_recent + 1, by_ratio))


def poison_padding(inp: BlockTopKInputs) -> int:
    """Fill the slots past each request's last token, in its last page, with
    NaN in K and V (their contents are unspecified; the kernels must weigh
    them by 0 without reading NaN into the output). Returns the slots set."""
    from workloads.generate import BF16_NAN_BITS
    P = inp.cfg.page_size
    nan = torch.tensor(BF16_NAN_BITS, dtype=torch.int16).view(torch.bfloat16).item()
    lens = inp.seq_lens.cpu().tolist()
    indptr = inp.page_indptr.cpu().tolist()
    idx = inp.page_indices.cpu().tolist()
    n = 0
    for r, L in enumerate(lens):
        if L % P:
            page = idx[indptr[r] + L // P]
            inp.k_pool[page, :, L % P:] = nan
            inp.v_pool[page, :, L % P:] = nan
            n += P - L % P
    return n


def build_summaries(inp: BlockTopKInputs, score_mode: str = "mean") -> torch.Tensor:
    """Block-mean summaries [pages][Hkv][D] or Quest bounds [pages][Hkv][2][D]
    of every complete page (other rows zero)."""
    import query_aware_sparse_ls_amd as ls
    dev = inp.k_pool.device
    Hkv, D = inp.cfg.num_kv_heads, inp.cfg.head_dim
    ids = complete_pages(inp).to(dev)
    if score_mode == "bounds":
        out = torch.zeros(inp.num_pages, Hkv, 2, D, dtype=torch.bfloat16, device=dev)
        return ls.build_block_bounds(inp.k_pool, ids, out)
    out = torch.zeros(inp.num_pages, Hkv, D, dtype=torch.bfloat16, device=dev)
    return ls.build_block_summaries(inp.k_pool, ids, out)


def run_gpu_step(inp: BlockTopKInputs, *, topk=None, n_sink=None, n_recent=None, agg=None,
                 out_dtype=None, keep_ratio=0.0, sm_scale=None, dense=False,
                 score_mode="mean") -> GpuStep:
    import query_aware_sparse_ls_amd as ls
    cfg = inp.cfg
    topk = inp.topk if topk is None else topk
    n_sink = cfg.n_sink if n_sink is None else n_sink
    n_recent = cfg.n_recent if n_recent is None else n_recent
    agg = cfg.group_agg if agg is None else agg
    out_dtype = out_dtype or (torch.float32 if cfg.out_dtype == "fp32" else torch.bfloat16)
    sm_scale = (1.0 / math.sqrt(cfg.head_dim)) if sm_scale is None else sm_scale
    dev = inp.k_pool.device
    B, Hq, D = inp.q.shape
    Hkv = cfg.num_kv_heads
    batch = paged_batch(inp)
    summ = build_summaries(inp, score_mode)
    maxsel = max_selected_for(topk, n_sink, n_recent, batch.max_blocks, keep_ratio)
    scores = torch.full((B, Hkv, batch.max_blocks), float("nan"), dtype=torch.float32, device=dev)
    sel, cnt = ls.score_select(inp.q, summ, cfg.page_size, batch, topk=topk, n_sink=n_sink,
                               n_recent=n_recent, max_selected=maxsel, group_agg=agg,
                               keep_ratio=keep_ratio, scores_out=scores, score_mode=score_mode)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    if dense:
        out, _ = ls.sparse_attn_decode(inp.q, inp.k_pool, inp.v_pool, batch, None, None,
                                       sm_scale=sm_scale, out_dtype=out_dtype, lse=lse)
    else:
        out, _ = ls.sparse_attn_decode(inp.q, inp.k_pool, inp.v_pool, batch, sel, cnt,
                                       sm_scale=sm_scale, out_dtype=out_dtype, lse=lse)
    torch.cuda.synchronize()
    return GpuStep(summ, scores, sel, cnt, out, lse)


def sub_problem(inp: BlockTopKInputs, r: int, g: int):
    """Request r, kv head g as a one-request, one-kv-head oracle problem with
    a contiguous page table (pages gathered on the device, then copied)."""
    P = inp.cfg.page_size
    G = inp.cfg.group
    L = int(inp.seq_lens[r])
    nb = -(-L // P)
    p0 = int(inp.page_indptr[r])
    pages = inp.page_indices[p0:p0 + nb].long()
    k = bf16_bits(inp.k_pool[pages, g:g + 1].contiguous())
    v = bf16_bits(inp.v_pool[pages, g:g + 1].contiguous())
    q = bf16_bits(inp.q[r:r + 1, g * G:(g + 1) * G].contiguous())
    batch = BatchView(np.array([0, nb]), np.arange(nb), np.array([L]), P)
    return q, k, v, batch


def check_selection(gpu_sel: List[int], scores: np.ndarray, nb: int, nc: int, k: int,
                    n_sink: int, n_recent: int) -> Dict:
    """GPU selection vs the oracle's, exact outside the near-tie band around
    the oracle's k-th candidate score; same size; ascending and unique."""
    want = oracle.select_blocks(scores, nb, nc, k, n_sink, n_recent)
    assert gpu_sel == sorted(set(gpu_sel)), "selection not ascending/unique"
    assert len(gpu_sel) == len(want), (len(gpu_sel), len(want))
    forced = set(forced_blocks(nb, nc, n_sink, n_recent))
    cands = [j for j in range(nc) if j not in forced]
    band = set()
    if 0 < k < len(cands):
        s = np.array([scores[j] for j in cands])
        sk = np.sort(s)[::-1][k - 1]
        tau = TIE_REL * abs(sk) + TIE_ABS_OF_MAX * np.max(np.abs(s))
        band = {j for j in cands if abs(scores[j] - sk) <= tau}
    assert forced <= set(gpu_sel)
    assert set(gpu_sel) - band == set(want) - band, (
        sorted(set(gpu_sel) ^ set(want)), sorted(band))
    return {"band": len(band), "want": want}


def check_pair(inp: BlockTopKInputs, res: GpuStep, r: int, g: int, *, topk, n_sink, n_recent,
               agg, sm_scale, out_dtype, check_scores=True, dense=False, score_mode="mean"):
    """Full parity of one (request, kv head): summaries (block means, or Quest
    bounds), scores, selection and attention output (oracle attention on the
    GPU's own selection)."""
    q, k, v, batch = sub_problem(inp, r, g)
    L = int(batch.seq_lens[0])
    nb, nc = batch.num_blocks(0), batch.num_complete(0)
    P = inp.cfg.page_size
    G = inp.cfg.group
    # summaries: bit-exact
    D = k.shape[-1]
    if score_mode == "bounds":
        summ = oracle.block_bounds(k, np.arange(nc))
    else:
        summ = oracle.block_summaries(k, np.arange(nc)) if nc else np.zeros((0, 1, D), np.uint16)
    p0 = int(inp.page_indptr[r])
    pages = inp.page_indices[p0:p0 + nc].long()
    gsum = bf16_bits(res.summaries[pages, g:g + 1].contiguous())
    assert np.array_equal(gsum, summ), "summaries differ"
    # scores (fp32 GPU vs fp64 oracle)
    if not nc:
        s = np.zeros(0)
    elif score_mode == "bounds":
        s = oracle.bound_scores(q, summ, batch, 0, 0, num_kv_heads=1, agg=agg)
    else:
        s = oracle.block_scores(q, summ, batch, 0, 0, num_kv_heads=1, agg=agg)
    forced = set(forced_blocks(nb, nc, n_sink, n_recent))
    cands = [j for j in range(nc) if j not in forced]
    if check_scores and cands and res.scores is not None:
        gs = res.scores[r, g, cands].double().cpu().numpy()
        np.testing.assert_allclose(gs, s[cands], rtol=1e-5, atol=1e-5 * max(1.0, np.abs(s).max()))
    cnt = int(res.counts[r, g])
    gsel = res.selected[r, g, :cnt].cpu().tolist()
    pad = res.selected[r, g, cnt:].cpu()
    assert bool((pad == -1).all()), "selection padding must be -1"
    if dense:
        gsel_eff = list(range(nb))
        info = {"band": 0}
    else:
        info = check_selection(gsel, s, nb, nc, topk, n_sink, n_recent)
        gsel_eff = gsel
    odt = "fp32" if out_dtype == torch.float32 else "bf16"
    o, lse = oracle.sparse_attention(q, k, v, batch, 0, 0, gsel_eff, num_kv_heads=1,
                                     sm_scale=np.float64(np.float32(sm_scale)), out_dtype="fp64")
    got = res.out[r, g * G:(g + 1) * G].float().cpu().numpy().astype(np.float64)
    if odt == "fp32":
        np.testing.assert_allclose(got, o, rtol=0, atol=FP32_ATOL)
    else:
        want16 = oracle.bf16_to_f64(oracle.f64_to_bf16_bits(o))
        np.testing.assert_allclose(got, want16, rtol=0, atol=BF16_ATOL)
        # and within a couple of bf16 ulps of the exact value
        np.testing.assert_allclose(got, o, rtol=1e-2, atol=2e-3)
    glse = res.lse[r, g * G:(g + 1) * G].double().cpu().numpy()
    fin = np.isfinite(lse)
    assert np.array_equal(np.isfinite(glse), fin)
    np.testing.assert_allclose(glse[fin], lse[fin], rtol=2e-6, atol=2e-5)
    return info


def run_gpu_fused(inp: BlockTopKInputs, *, topk=None, n_sink=None, n_recent=None, agg=None,
                  out_dtype=None, keep_ratio=0.0, sm_scale=None, workspace=None,
                  summaries=None, new_pages=None, score_mode="mean") -> GpuStep:
    """The whole step in one call (ls_sparse_decode_step); it keeps its
    block scores on chip, so the result carries none."""
    import query_aware_sparse_ls_amd as ls
    cfg = inp.cfg
    topk = inp.topk if topk is None else topk
    n_sink = cfg.n_sink if n_sink is None else n_sink
    n_recent = cfg.n_recent if n_recent is None else n_recent
    agg = cfg.group_agg if agg is None else agg
    out_dtype = out_dtype or (torch.float32 if cfg.out_dtype == "fp32" else torch.bfloat16)
    sm_scale = (1.0 / math.sqrt(cfg.head_dim)) if sm_scale is None else sm_scale
    dev = inp.k_pool.device
    B, Hq, D = inp.q.shape
    Hkv = cfg.num_kv_heads
    batch = paged_batch(inp)
    if summaries is None:
        summaries = build_summaries(inp, score_mode)
    maxsel = max_selected_for(topk, n_sink, n_recent, batch.max_blocks, keep_ratio)
    if workspace is None:
        workspace = ls.sparse_decode_step_workspace(B, Hq, Hkv, D, batch.max_blocks, maxsel, dev)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    out, _, sel, cnt = ls.sparse_decode_step(
        inp.q, summaries, inp.k_pool, inp.v_pool, batch, topk=topk, n_sink=n_sink,
        n_recent=n_recent, max_selected=maxsel, sm_scale=sm_scale, group_agg=agg,
        keep_ratio=keep_ratio, out_dtype=out_dtype, lse=lse, new_pages=new_pages,
        workspace=workspace, score_mode=score_mode)
    torch.cuda.synchronize()
    return GpuStep(summaries, None, sel, cnt, out, lse)
