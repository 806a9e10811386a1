"""The streaming-read ceiling kernel (benchmark instrumentation) reads every
32-bit word of its range exactly once: the XOR of its per-block folds equals
numpy's, for grids that split the range raggedly (a word read twice or missed
changes the XOR), including blocks left without a piece (they write 0)."""
import numpy as np
import pytest
import torch

from kv_cache_reads_amd import rma as R

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_words,blocks", [(4, 1), (4100, 7), (1 << 20, 512), ((1 << 20) + 4 * 333, 512),
                                            (3 * 4096 + 4, 4096)])
def test_stream_read_xor_covers_every_word_once(n_words, blocks):
    g = torch.Generator().manual_seed(n_words + blocks)
    x = torch.randint(-2**31, 2**31 - 1, (n_words,), generator=g, dtype=torch.int64).to(torch.int32)
    want = int(np.bitwise_xor.reduce(x.numpy().view(np.uint32)))
    xd = x.cuda()
    sink = torch.full((blocks + 1,), 12345, dtype=torch.int32, device="cuda")
    R.rma_stream_read(xd, blocks, sink)
    torch.cuda.synchronize()
    folds = sink.cpu().numpy().view(np.uint32)
    assert int(np.bitwise_xor.reduce(folds[:blocks])) == want
    assert folds[blocks] == 12345   # nothing past the grid's words
