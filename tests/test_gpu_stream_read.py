"""The measuring stick rq_stream_read reads every 16-byte unit of the buffer it is given once:
with the sink cleared, the XOR of all sink words equals the XOR of every 32-bit word of the
buffer (random contents, so a unit skipped or read twice changes the fold).  Sizes cover one
unit, a ragged tail within a workgroup's slab, and a buffer split over every workgroup (two per CU)."""
import numpy as np
import pytest
import torch

from _support import say

pytestmark = pytest.mark.gpu

SINK_WORDS = 4096 * 256


@pytest.mark.parametrize("nbytes", [16, 48 * 1024 + 16, 3 * 1024 * 1024 + 4096 + 16, 96 * 1024 * 1024])
def test_stream_read_folds_every_word(nbytes):
    from looped_transformer_decode_amd import binding as B
    say(f"[stream_read] bytes={nbytes}")
    dev = torch.device("cuda:0")
    g = torch.Generator().manual_seed(nbytes % 1000003)
    host = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g)
    buf = host.to(dev)
    sink = torch.zeros(SINK_WORDS, dtype=torch.int32, device=dev)
    B.rq_stream_read(buf, nbytes, sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want, f"fold {got:#010x} != {want:#010x}"
    # a prefix of the buffer folds to the prefix's words only
    part = nbytes // 2 // 16 * 16 or 16
    sink.zero_()
    B.rq_stream_read(buf, part, sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host.numpy()[:part // 4].view(np.uint32))
    assert np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)) == want
