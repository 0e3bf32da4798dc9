"""GPU parity of GQA groups other than 4 (1, 2 and 8 query heads per KV head)
on the block path: block scores aggregated over the group (Vortex post, the
GQA-grouped block scoring of "Writing an algorithm: vFlow"), the top-k with
forced blocks, and attention over the selected blocks (the block top-k
equation of "Why Long Generations Are Expensive"), against the float64
oracle, pair by pair; the dense (k = all) path; the whole step in one call,
bit-identical to the separate calls, with the summary refresh of pages that
just filled.
"""

import math

import pytest
import torch

from parity_util import build_summaries, check_pair, run_gpu_fused, run_gpu_step, say
from workloads import LLAMA8B_32K_B16, make_block_topk_inputs, reduced

pytestmark = pytest.mark.gpu

# (group, q heads, kv heads)
GROUPS = [(1, 8, 8), (2, 16, 8), (8, 32, 4)]
LENS = [5000, 1234, 17, 4096]   # ragged: a partial last page, a tiny request, whole pages


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _cfg(G, hq, hkv, D, **kw):
    return reduced(LLAMA8B_32K_B16, name=f"gqa{G}_d{D}", batch=len(LENS), num_q_heads=hq,
                   num_kv_heads=hkv, head_dim=D, context=max(LENS), topk=24, **kw)


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


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("G,hq,hkv", GROUPS, ids=[f"g{g[0]}" for g in GROUPS])
@pytest.mark.parametrize("agg,out_dtype", [("max", "fp32"), ("mean", "bf16")])
def test_groups_select_and_attend(G, hq, hkv, D, agg, out_dtype):
    cfg = _cfg(G, hq, hkv, D, group_agg=agg, out_dtype=out_dtype)
    say(f"GQA group {G}: {cfg.name}, lens {LENS}, agg {agg}, out {out_dtype}")
    inp = make_block_topk_inputs(cfg, device="cuda", seed=90 + G, seq_lens=LENS)
    assert inp.cfg.group == G
    res = run_gpu_step(inp)
    for r in range(cfg.batch):
        for g in range(hkv):
            check_pair(inp, res, r, g, **_kw(inp))


@pytest.mark.parametrize("G,hq,hkv", GROUPS, ids=[f"g{g[0]}" for g in GROUPS])
def test_groups_dense(G, hq, hkv):
    cfg = _cfg(G, hq, hkv, 128)
    say(f"GQA group {G}, dense: {cfg.name}")
    inp = make_block_topk_inputs(cfg, device="cuda", seed=95 + G, seq_lens=LENS)
    res = run_gpu_step(inp, dense=True)
    for r in range(cfg.batch):
        for g in (0, hkv - 1):
            check_pair(inp, res, r, g, dense=True, check_scores=False, **_kw(inp))


@pytest.mark.parametrize("G,hq,hkv", GROUPS, ids=[f"g{g[0]}" for g in GROUPS])
def test_groups_fused_step_with_refresh(G, hq, hkv):
    """The step in one call equals the separate calls bit for bit, and with
    every request's last complete page stale (NaN) and passed as just filled,
    it rebuilds those summaries and still gives the same result."""
    cfg = _cfg(G, hq, hkv, 128)
    say(f"GQA group {G}, fused step: {cfg.name}")
    inp = make_block_topk_inputs(cfg, device="cuda", seed=97 + G, seq_lens=LENS)
    sep = run_gpu_step(inp)
    fus = run_gpu_fused(inp, summaries=sep.summaries)
    _same(sep, fus)
    P = cfg.page_size
    indptr = inp.page_indptr.cpu().tolist()
    idx = inp.page_indices.cpu()
    new = [int(idx[indptr[r] + L // P - 1]) for r, L in enumerate(LENS) if L >= 2 * P]
    new = torch.tensor(new, dtype=torch.int32, device="cuda")
    stale = sep.summaries.clone()
    stale[new.long()] = float("nan")
    ref = run_gpu_fused(inp, summaries=build_summaries(inp))
    got = run_gpu_fused(inp, summaries=stale, new_pages=new)
    assert torch.equal(stale.view(torch.int16), sep.summaries.view(torch.int16))
    _same(ref, got)
    for r in range(cfg.batch):
        check_pair(inp, got, r, 0, check_scores=False, **_kw(inp))


def test_group8_full_size_16x32k_sampled():
    """64 query heads over 8 kv heads (group 8) at 16 requests x 32K: the
    split kernels at the benchmark's batch and context; sampled pairs against
    the oracle, every pair's selection size and padding checked."""
    cfg = reduced(LLAMA8B_32K_B16, name="gqa8_16x32k", num_q_heads=64, num_kv_heads=8)
    say(f"GQA group 8 at full size: {cfg.name}")
    inp = make_block_topk_inputs(cfg, device="cuda", seed=99)
    res = run_gpu_step(inp)
    nb = cfg.context // cfg.page_size
    want = min(nb, inp.topk + cfg.n_sink + cfg.n_recent)
    assert (res.counts == want).all()
    for r, g in [(0, 0), (5, 3), (11, 6), (15, 7)]:
        check_pair(inp, res, r, g, **_kw(inp))
