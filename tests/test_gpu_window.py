"""GPU parity of the sink + recent window attention (ls_window_attn_decode):
the first n_sink tokens and the last `window` tokens of every request, read
in place, against the oracle's softmax over that token set. Outputs within
1e-5 (fp32) or 2e-2 (bf16), lse within 2e-6 relative; two calls
bit-identical.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from parity_util import BF16_ATOL, FP32_ATOL, paged_batch, poison_padding, say, sub_problem
from workloads import LLAMA8B_32K_B16, TINY_4K, make_block_topk_inputs, reduced

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(inp, n_sink, window, out_dtype):
    import query_aware_sparse_ls_amd as ls
    B, Hq, D = inp.q.shape
    lse = torch.empty(B, Hq, dtype=torch.float32, device=inp.q.device)
    out, _ = ls.window_attn_decode(inp.q, inp.k_pool, inp.v_pool, paged_batch(inp), n_sink=n_sink,
                                   window=window, sm_scale=1.0 / math.sqrt(D),
                                   out_dtype=out_dtype, lse=lse)
    torch.cuda.synchronize()
    return out, lse


def _check(inp, out, lse, r, g, n_sink, window, out_dtype):
    G = inp.cfg.group
    q, k, v, batch = sub_problem(inp, r, g)
    sm = np.float64(np.float32(1.0 / math.sqrt(inp.cfg.head_dim)))
    o, want_lse = oracle.window_attention(q, k, v, batch, 0, 0, n_sink=n_sink, window=window,
                                          num_kv_heads=1, sm_scale=sm, out_dtype="fp64")
    got = out[r, g * G:(g + 1) * G].double().cpu().numpy()
    if out_dtype == torch.float32:
        np.testing.assert_allclose(got, o, rtol=0, atol=FP32_ATOL)
    else:
        want16 = oracle.bf16_to_f64(oracle.f64_to_bf16_bits(o))
        np.testing.assert_allclose(got, want16, rtol=0, atol=BF16_ATOL)
    glse = lse[r, g * G:(g + 1) * G].double().cpu().numpy()
    fin = np.isfinite(want_lse)
    assert np.array_equal(np.isfinite(glse), fin)
    np.testing.assert_allclose(glse[fin], want_lse[fin], rtol=2e-6, atol=2e-5)


@pytest.mark.parametrize("n_sink,window", [(4, 1000), (4, 30), (0, 500), (4, 0), (20, 9),
                                           (4, 10), (100, 4000)])
def test_window_ragged_lengths(n_sink, window):
    """Ragged lengths: empty, shorter than the sinks, ranges that touch, a
    gap inside one block (the block read twice), and NaN in the unused
    slots of partial pages."""
    lens = [5000, 0, 3, 12, 14, 16, 17, 30, 33, 100, 1024, 4097, 2500, 777, 64, 9999]
    cfg = reduced(LLAMA8B_32K_B16, context=max(lens))
    say(f"window attention: n_sink {n_sink}, window {window}")
    inp = make_block_topk_inputs(cfg, device="cuda", seed=81, seq_lens=lens)
    poison_padding(inp)
    out, lse = _run(inp, n_sink, window, torch.float32)
    out2, lse2 = _run(inp, n_sink, window, torch.float32)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    for r in range(len(lens)):
        _check(inp, out, lse, r, (3 * r) % cfg.num_kv_heads, n_sink, window, torch.float32)


def test_window_d64_bf16():
    cfg = reduced(TINY_4K, batch=4, context=3000)
    inp = make_block_topk_inputs(cfg, device="cuda", seed=82)
    out, lse = _run(inp, 4, 700, torch.bfloat16)
    for r in range(4):
        for g in range(cfg.num_kv_heads):
            _check(inp, out, lse, r, g, 4, 700, torch.bfloat16)


def test_window_full_size_llama8b_32k_b16():
    """The bench's window call: 4 sinks and the last 9,830 tokens (30% of
    32K) of 16 requests, sampled pairs."""
    cfg = LLAMA8B_32K_B16
    inp = make_block_topk_inputs(cfg, device="cuda")
    out, lse = _run(inp, 4, 9830, torch.bfloat16)
    for r, g in [(0, 0), (2, 5), (5, 1), (7, 3), (9, 6), (11, 2), (13, 4), (15, 7)]:
        _check(inp, out, lse, r, g, 4, 9830, torch.bfloat16)
