"""moe_stream_read through the C ABI: every 16-byte piece of the buffer is
read exactly once, so the XOR of the per-thread words equals the XOR of all
words of the buffer, for grids that do and do not divide the piece count."""
import numpy as np
import pytest
import torch

from sparse_mixture_experts_amd import moe

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("pieces,blocks", [(1, 1), (37, 1), (4096 * 7 + 5, 13), (1 << 16, 256)])
def test_stream_read_reads_every_word_once(pieces, blocks):
    rng = np.random.default_rng(pieces)
    host = rng.integers(0, 2**32, size=pieces * 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to("cuda:0")
    out = torch.empty(blocks * 256, dtype=torch.int32, device="cuda:0")
    moe.moe_stream_read(src, pieces * 16, out, blocks)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(host))
