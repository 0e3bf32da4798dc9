"""The stream-read reference kernel (ls_stream_read): it reads every word of
the buffer (the XOR of the sink words equals the XOR of all 32-bit words,
computed on the host), at a size that is not a multiple of one grid pass."""

import numpy as np
import pytest
import torch

from parity_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("nbytes", [16, 4096 * 256 * 16 * 4 + 48, 137_658_368])
def test_stream_read_reads_every_word(nbytes):
    import query_aware_sparse_ls_amd as ls
    say(f"stream read of {nbytes} bytes")
    g = torch.Generator(device="cpu").manual_seed(nbytes % 1000)
    host = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), generator=g, dtype=torch.int64)
    host = host.to(torch.int32)
    src = host.cuda()
    sink = ls.stream_read(src)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert int(got) == int(want)
