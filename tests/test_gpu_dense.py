"""GPU parity of the k = all (dense) path: ls_sparse_attn_decode with no
selection, split-K over runs of consecutive blocks of each (request, kv head)
pair, against the oracle's attention over every token of the request.

Outputs within 2e-2 (bf16, also against the oracle rounded to bf16) or 1e-5
(fp32); lse within 2e-6 relative; two calls bit-identical.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from parity_util import BF16_ATOL, FP32_ATOL, paged_batch, poison_padding, say, sub_problem
from workloads import LLAMA8B_32K_B16, make_block_topk_inputs, reduced

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import query_aware_sparse_ls_amd as ls
    say("libls:", ls.version(), ls._lib.LIB_PATH)


def _dense(inp, out_dtype):
    import query_aware_sparse_ls_amd as ls
    B, Hq, D = inp.q.shape
    lse = torch.empty(B, Hq, dtype=torch.float32, device=inp.q.device)
    out, _ = ls.sparse_attn_decode(inp.q, inp.k_pool, inp.v_pool, paged_batch(inp), None, None,
                                   sm_scale=1.0 / math.sqrt(D), out_dtype=out_dtype, lse=lse)
    torch.cuda.synchronize()
    return out, lse


def _check(inp, out, lse, r, g, out_dtype):
    G = inp.cfg.group
    q, k, v, batch = sub_problem(inp, r, g)
    sm = np.float64(np.float32(1.0 / math.sqrt(inp.cfg.head_dim)))
    o, want_lse = oracle.dense_attention(q, k, v, batch, 0, 0, num_kv_heads=1, sm_scale=sm,
                                         out_dtype="fp64")
    got = out[r, g * G:(g + 1) * G].double().cpu().numpy()
    if out_dtype == torch.float32:
        np.testing.assert_allclose(got, o, rtol=0, atol=FP32_ATOL)
    else:
        want16 = oracle.bf16_to_f64(oracle.f64_to_bf16_bits(o))
        np.testing.assert_allclose(got, want16, rtol=0, atol=BF16_ATOL)
        np.testing.assert_allclose(got, o, rtol=1e-2, atol=2e-3)
    glse = lse[r, g * G:(g + 1) * G].double().cpu().numpy()
    fin = np.isfinite(want_lse)
    assert np.array_equal(np.isfinite(glse), fin)
    np.testing.assert_allclose(glse[fin], want_lse[fin], rtol=2e-6, atol=2e-5)
    if not fin.any():
        assert not got.any(), "an empty request must give zeros"


def _pairs(cfg, n, seed=0):
    rng = np.random.default_rng(seed)
    allp = [(r, g) for r in range(cfg.batch) for g in range(cfg.num_kv_heads)]
    pick = {allp[0], allp[-1]}
    for i in rng.permutation(len(allp))[:n]:
        pick.add(allp[int(i)])
    return sorted(pick)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_dense_full_size_llama8b_32k_b16(out_dtype):
    """The bench's dense call (16 requests x 32K, 128 pairs, 16 runs of 128
    blocks each), sampled pairs against the oracle; a second call is
    bit-identical."""
    cfg = LLAMA8B_32K_B16
    say(f"dense at full size: {cfg.name}, out {out_dtype}")
    inp = make_block_topk_inputs(cfg, device="cuda")
    out, lse = _dense(inp, out_dtype)
    out2, lse2 = _dense(inp, out_dtype)
    assert torch.equal(out, out2) and torch.equal(lse, lse2), "run-to-run determinism"
    for r, g in [(0, 0), (7, 3), (15, 7)]:
        _check(inp, out, lse, r, g, out_dtype)


def test_dense_longest_runs_ragged_lengths():
    """Runs of the maximum 512 blocks (256 pairs at head_dim 64, up to 4,097
    blocks), with a one-block tail run and requests that are empty, a
    fraction of a page, or end inside their last run."""
    lens = [65541, 0, 1, 15, 16, 17, 8191, 8192, 8193, 65536, 40000, 33, 511 * 16 + 3,
            512 * 16, 512 * 16 + 1, 30000]
    lens = (lens * 2)[:32]
    cfg = reduced(LLAMA8B_32K_B16, batch=32, num_q_heads=32, num_kv_heads=8, head_dim=64,
                  context=max(lens))
    say(f"dense ragged, runs of 512 blocks: {cfg.name} lens {lens[:16]}")
    inp = make_block_topk_inputs(cfg, device="cuda", seed=61, seq_lens=lens)
    out, lse = _dense(inp, torch.float32)
    pairs = [(0, 0), (1, 2), (2, 5), (3, 1), (5, 7), (8, 4), (12, 3), (14, 6), (31, 7)]
    for r, g in pairs:
        _check(inp, out, lse, r, g, torch.float32)


def test_dense_one_request_many_runs():
    """8 pairs over 100,000 tokens: about 2,048 workgroups of 32-block runs,
    bf16 output."""
    cfg = reduced(LLAMA8B_32K_B16, batch=1, context=100000)
    say(f"dense, one request, many runs: {cfg.name}")
    inp = make_block_topk_inputs(cfg, device="cuda", seed=62)
    out, lse = _dense(inp, torch.bfloat16)
    for g in range(cfg.num_kv_heads):
        _check(inp, out, lse, 0, g, torch.bfloat16)


def test_dense_nan_in_unused_pages_stays_out():
    """Pages outside every request's page list, and the slots past each
    request's last token, hold NaN: outputs stay finite and exact."""
    cfg = reduced(LLAMA8B_32K_B16, batch=4, context=5000, page_table="pool",
                  pool_occupancy=0.5)
    say(f"dense with NaN-poisoned unused pages: {cfg.name}")
    inp = make_block_topk_inputs(cfg, device="cuda", seed=63, poison_unused=True)
    assert poison_padding(inp) > 0
    out, lse = _dense(inp, torch.float32)
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    for r, g in _pairs(cfg, 6):
        _check(inp, out, lse, r, g, torch.float32)
