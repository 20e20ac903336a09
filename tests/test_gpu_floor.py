"""dsel_read_floor (the streaming-read floor helper) reads every byte once:
its per-64-KiB-block XOR words match the same fold on the host, for sizes
with and without a partial last block."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsel():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_indexer_dsel_amd as d
    return d


@pytest.mark.parametrize("nbytes", [16, 65536, 65536 * 3 + 48, 66191360])
def test_read_floor_reads_every_byte(dsel, nbytes):
    g = torch.Generator().manual_seed(nbytes % 1000 + 7)
    host = torch.randint(-(1 << 31), 1 << 31, (nbytes // 4,), dtype=torch.int64, generator=g).to(torch.int32)
    words = dsel.read_floor(host.cuda()).cpu().numpy().view(np.uint32)
    h = host.numpy().view(np.uint32)
    blocks = -(-nbytes // 65536)
    pad = np.zeros(blocks * 16384, dtype=np.uint32)
    pad[:h.size] = h
    want = np.bitwise_xor.reduce(pad.reshape(blocks, 16384), axis=1)
    assert words.shape == (blocks,)
    assert (words == want).all()
