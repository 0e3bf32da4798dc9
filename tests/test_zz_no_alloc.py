"""ls_sparse_decode_step_noalloc (the step with the library's fixed scratch
array instead of a caller workspace) gives the same bits as
ls_sparse_decode_step, call after call on the one shared array, the second
call with a smaller input; shapes on the per-pair route (no scratch used) and
on the many-workgroups and planned routes (scratch used: control words,
scores, selection entries, split states)."""

import math

import pytest
import torch

from parity_util import paged_batch, run_gpu_step, say
from workloads import LLAMA8B_32K_B16, make_block_topk_inputs, reduced

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _both(inp, summaries):
    import query_aware_sparse_ls_amd as ls
    cfg = inp.cfg
    B, Hq, D = inp.q.shape
    Hkv = cfg.num_kv_heads
    batch = paged_batch(inp)
    maxsel = min(batch.max_blocks, inp.topk + cfg.n_sink + cfg.n_recent + 1)
    kw = dict(topk=inp.topk, n_sink=cfg.n_sink, n_recent=cfg.n_recent, max_selected=maxsel,
              sm_scale=1.0 / math.sqrt(D))
    outs = []
    for noalloc in (False, True):
        sel = torch.full((B, Hkv, maxsel), -7, dtype=torch.int32, device="cuda")
        cnt = torch.full((B, Hkv), -7, dtype=torch.int32, device="cuda")
        out = torch.full((B, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            ls.sparse_decode_step_noalloc(inp.q, summaries, inp.k_pool, inp.v_pool, batch,
                                          selected=sel, selected_count=cnt, out=out, lse=lse,
                                          **kw)
        else:
            ls.sparse_decode_step(inp.q, summaries, inp.k_pool, inp.v_pool, batch, selected=sel,
                                  selected_count=cnt, out=out, lse=lse, **kw)
        torch.cuda.synchronize()
        outs.append((sel, cnt, out, lse))
    (s0, c0, o0, l0), (s1, c1, o1, l1) = outs
    assert torch.equal(c0, c1)
    for r in range(B):
        for g in range(Hkv):
            n = int(c0[r, g])
            assert torch.equal(s0[r, g, :n], s1[r, g, :n])
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(l0, l1)


@pytest.mark.parametrize("route,first,second", [
    # 16 and 8 (request, kv head) pairs: the many-workgroups route, scratch in use
    ("flow", dict(batch=2, context=4096 + 7), dict(batch=1, context=2500)),
    # 128 and 64 pairs of at most 4096 blocks: one workgroup per pair
    ("per-pair", dict(batch=16, context=3000), dict(batch=8, context=1100)),
    # 64 pairs of more than 4096 blocks: the planned route (score rows, split
    # states of pairs cut by range ends, arrival counters in scratch)
    ("planned", dict(batch=8, context=70000), dict(batch=8, context=66000)),
])
def test_noalloc_matches_step_two_calls(route, first, second):
    for i, shape in enumerate((first, second)):
        cfg = reduced(LLAMA8B_32K_B16, **shape)
        say(f"no-alloc step vs workspace step, {route} route, call {i}: {cfg.name}")
        inp = make_block_topk_inputs(cfg, device="cuda", seed=40 + i)
        ref = run_gpu_step(inp)
        _both(inp, ref.summaries)
