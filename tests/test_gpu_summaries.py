"""ls_build_block_summaries and ls_build_block_bounds on bf16 key pools of
every supported geometry (head_dim 64 / 128, page_size 16 / 32 / 64, bf16 /
fp32 summaries): bit-exact against the oracle's exact-sum means and bounds,
rows of unlisted pages untouched, and a full-size build (16 x 32K keys)."""

import numpy as np
import pytest
import torch

import oracle
from parity_util import say
from workloads import bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _keys(num_pages, H, P, D, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    k = torch.randn(num_pages, H, P, D, generator=g) * 3
    k[:, :, 0, :5] = 1e-3          # columns whose terms span many binades
    k[1, 0, :, 7] = 2.0 ** 60      # a huge term next to small ones
    return k.to(torch.bfloat16).cuda()


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("P", [16, 32, 64])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_summaries_bit_exact(D, P, out_dtype):
    import query_aware_sparse_ls_amd as ls
    say(f"summaries D {D} P {P} {out_dtype}")
    num_pages, H = 37, 3
    k = _keys(num_pages, H, P, D, seed=D + P)
    ids = torch.tensor([5, 0, 36, 1, 17, 9], dtype=torch.int32, device="cuda")
    out = torch.full((num_pages, H, D), 7.0, dtype=out_dtype, device="cuda")
    ls.build_block_summaries(k, ids, out)
    torch.cuda.synchronize()
    want = oracle.block_summaries(bf16_bits(k), ids.cpu().numpy(),
                                  out_dtype="bf16" if out_dtype == torch.bfloat16 else "fp32")
    got = out[ids.long()].cpu()
    if out_dtype == torch.bfloat16:
        assert np.array_equal(bf16_bits(got), want)
    else:
        assert np.array_equal(got.numpy().view(np.uint32), np.asarray(want, dtype=np.float32).view(np.uint32))
    rest = [p for p in range(num_pages) if p not in set(ids.tolist())]
    assert (out[rest].float() == 7.0).all()


@pytest.mark.parametrize("D,P", [(128, 64), (64, 32)])
def test_bounds_other_geometries_bit_exact(D, P):
    import query_aware_sparse_ls_amd as ls
    num_pages, H = 20, 2
    k = _keys(num_pages, H, P, D, seed=3 * D + P)
    ids = torch.tensor([19, 3, 0, 11], dtype=torch.int32, device="cuda")
    out = torch.zeros(num_pages, H, 2, D, dtype=torch.bfloat16, device="cuda")
    ls.build_block_bounds(k, ids, out)
    torch.cuda.synchronize()
    want = oracle.block_bounds(bf16_bits(k), ids.cpu().numpy())
    assert np.array_equal(bf16_bits(out[ids.long()].cpu()), want)


def test_full_size_build_llama8b_32k_b16():
    """Every complete page of 16 x 32K tokens (8 KV heads, D 128): sampled
    pages bit-exact against the oracle."""
    import query_aware_sparse_ls_amd as ls
    num_pages, H, P, D = 16 * 2048, 8, 16, 128
    g = torch.Generator(device="cuda").manual_seed(5)
    k = torch.randn(num_pages, H, P, D, generator=g, device="cuda").to(torch.bfloat16)
    ids = torch.randperm(num_pages, device="cuda").to(torch.int32)
    out = torch.zeros(num_pages, H, D, dtype=torch.bfloat16, device="cuda")
    ls.build_block_summaries(k, ids, out)
    torch.cuda.synchronize()
    sample = np.array([0, 1, 777, 12345, num_pages - 1])
    want = oracle.block_summaries(bf16_bits(k[torch.as_tensor(sample, device="cuda")].contiguous()),
                                  np.arange(len(sample)))
    assert np.array_equal(bf16_bits(out[torch.as_tensor(sample, device="cuda")].contiguous()), want)
