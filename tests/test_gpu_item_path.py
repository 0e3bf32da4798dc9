"""GPU parity of the per-(request, kv head) kernels, which the library uses
when a call has at least 64 (request, kv head) pairs: one workgroup runs a
pair's scoring, top-k and attention with every intermediate on chip.

Same bar as the split kernels: selections equal to the oracle's outside the
near-tie band, outputs within 2e-2 (bf16) / 1e-5 (fp32) of the oracle's
attention over the GPU selection; the one-call step must equal the two
separate calls bit for bit.
"""

import math

import numpy as np
import pytest
import torch

from parity_util import check_pair, poison_padding, run_gpu_fused, run_gpu_step, say
from oracle.method import topk_from_keep_ratio
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


def _pairs(cfg, n, seed=0):
    """n (request, kv head) pairs spread over the batch, always with the
    first and the last."""
    rng = np.random.default_rng(seed)
    allp = [(r, g) for r in range(cfg.batch) for g in range(cfg.num_kv_heads)]
    pick = {allp[0], allp[-1]}
    for i in rng.permutation(len(allp))[:n]:
        pick.add(allp[int(i)])
    return sorted(pick)


def _same(a, b):
    assert torch.equal(a.counts, b.counts)
    for r in range(a.counts.shape[0]):
        for g in range(a.counts.shape[1]):
            n = int(a.counts[r, g])
            assert torch.equal(a.selected[r, g, :n], b.selected[r, g, :n])
    assert torch.equal(a.out, b.out)
    assert torch.equal(a.lse, b.lse)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("agg", ["max", "mean"])
def test_item_path_d64_many_pairs(agg, out_dtype):
    cfg = reduced(TINY_4K, batch=32)            # 64 pairs, head_dim 64
    say(f"per-pair kernels, d64, 64 pairs: agg={agg} out={out_dtype}")
    inp = make_block_topk_inputs(cfg, device="cuda", seed=41)
    sep = run_gpu_step(inp, agg=agg, out_dtype=out_dtype)
    fus = run_gpu_fused(inp, agg=agg, out_dtype=out_dtype, summaries=sep.summaries)
    _same(sep, fus)
    for r, g in _pairs(cfg, 10):
        check_pair(inp, sep, r, g, **_kw(inp, agg=agg, out_dtype=out_dtype))


@pytest.mark.parametrize("L", [1, 17, 33, 200, 1000])
def test_item_path_short_and_edge_lengths(L):
    cfg = reduced(TINY_4K, batch=32, context=L, n_hot=0)
    say(f"per-pair kernels, every request L={L}")
    inp = make_block_topk_inputs(cfg, device="cuda", seed=200 + L)
    for topk, ns, nr in ((0, 1, 1), (3, 1, 1), (2, 0, 0)):
        res = run_gpu_step(inp, topk=topk, n_sink=ns, n_recent=nr)
        fus = run_gpu_fused(inp, topk=topk, n_sink=ns, n_recent=nr, summaries=res.summaries)
        _same(res, fus)
        for r, g in _pairs(cfg, 4, seed=L):
            check_pair(inp, res, r, g, **_kw(inp, topk=topk, n_sink=ns, n_recent=nr))


def test_item_path_dense_k_all():
    cfg = reduced(LLAMA8B_32K_B16, batch=8, context=3000)   # 64 pairs
    say("per-pair dense attention (selection = every block)")
    inp = make_block_topk_inputs(cfg, device="cuda", seed=12)
    res = run_gpu_step(inp, dense=True, out_dtype=torch.float32)
    for r, g in _pairs(cfg, 8):
        check_pair(inp, res, r, g, **_kw(inp, dense=True, out_dtype=torch.float32))


@pytest.mark.parametrize("ratio", [1 / 16, 1.0])
def test_item_path_ragged_keep_ratio(ratio):
    cfg = reduced(RAGGED_B64, batch=8, ragged_range=(300, 70000))   # up to 4375 blocks
    say(f"per-pair kernels, ragged lengths, keep ratio {ratio}")
    inp = make_block_topk_inputs(cfg, device="cuda", seed=22)
    res = run_gpu_step(inp, topk=-1, keep_ratio=ratio)
    fus = run_gpu_fused(inp, topk=-1, keep_ratio=ratio, summaries=res.summaries)
    _same(res, fus)
    P = cfg.page_size
    lens = inp.seq_lens.tolist()
    for r, g in _pairs(cfg, 6, seed=3):
        L = lens[r]
        k = topk_from_keep_ratio(-(-L // P), L // P, ratio, cfg.n_sink, cfg.n_recent)
        check_pair(inp, res, r, g, **_kw(inp, topk=k))


def test_item_path_poisoned_unused_pages():
    cfg = reduced(RAGGED_B64, batch=8, ragged_range=(100, 6000), topk=8, keep_ratio=None,
                  pool_occupancy=0.7)
    say("per-pair kernels, NaN-poisoned unused pool pages and page padding")
    inp = make_block_topk_inputs(cfg, device="cuda", poison_unused=True)
    assert poison_padding(inp) > 0
    res = run_gpu_step(inp)
    assert torch.isfinite(res.out.float()).all()
    _same(res, run_gpu_fused(inp, summaries=res.summaries))
    for r, g in _pairs(cfg, 6, seed=4):
        check_pair(inp, res, r, g, **_kw(inp))


def test_item_path_ties_go_to_lowest_index():
    cfg = reduced(TINY_4K, batch=32, context=2048, n_hot=0)
    say("per-pair kernels, identical pages: lowest block indices win")
    inp = make_block_topk_inputs(cfg, device="cuda", seed=6)
    inp.k_pool[:] = inp.k_pool[0:1].clone()
    res = run_gpu_step(inp, topk=5, n_sink=1, n_recent=1)
    nb = 2048 // 16
    for r in range(cfg.batch):
        for g in range(cfg.num_kv_heads):
            got = res.selected[r, g, :int(res.counts[r, g])].tolist()
            assert got == [0, 1, 2, 3, 4, 5, nb - 1], got


@pytest.mark.parametrize("name,cfg", [
    ("d128 128 pairs", reduced(LLAMA8B_32K_B16, batch=16, context=100000)),
    ("d64 64 pairs", reduced(TINY_4K, batch=32, context=70000, n_hot=40, out_dtype="bf16")),
])
def test_pair_path_long_requests(name, cfg):
    """Requests of more than 4096 blocks in batches of at most 256 pairs take
    two workgroups per pair (split scoring, interleaved attention positions,
    merged softmax states): oracle parity and step == separate calls."""
    say(f"two workgroups per pair: {name}, L={cfg.context}")
    inp = make_block_topk_inputs(cfg, device="cuda", seed=77)
    res = run_gpu_step(inp)
    fus = run_gpu_fused(inp, summaries=res.summaries)
    _same(res, fus)
    for r, g in _pairs(cfg, 5, seed=5):
        check_pair(inp, res, r, g, **_kw(inp))
