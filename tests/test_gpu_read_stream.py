"""The streaming read behind the bench's read ceiling (ns_read_stream): every
byte of the buffer is read once -- the XOR of the workgroups' words equals the
XOR of all 32-bit words of the buffer, for a single chunk, a size that is no
multiple of the grid's stride and a large buffer -- and bad arguments are
refused."""
import numpy as np
import pytest
import torch

from decode_step_06_amd import ns
from gpu_helpers import say

pytestmark = pytest.mark.gpu

W = ns.NS_READ_STREAM_WORDS


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 64 << 20])
def test_read_stream_reads_every_word(nbytes):
    say(f"  read stream over {nbytes} bytes")
    g = torch.Generator().manual_seed(nbytes)
    host = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g)
    src = host.cuda()
    sink = torch.zeros(W, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()  # the buffers above were written on torch's stream
    ns.ns_read_stream(src.data_ptr(), nbytes, sink.data_ptr(), W, stream)
    stream.synchronize()
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want


def test_read_stream_rejects_bad_arguments():
    src = torch.zeros(64, dtype=torch.int32, device="cuda")
    sink = torch.zeros(W, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    bad = [
        (0, 16, sink.data_ptr(), W),                  # null source
        (src.data_ptr(), 16, 0, W),                   # null sink
        (src.data_ptr(), 0, sink.data_ptr(), W),      # nothing to read
        (src.data_ptr(), 20, sink.data_ptr(), W),     # not whole 16-byte chunks
        (src.data_ptr() + 4, 16, sink.data_ptr(), W),  # misaligned
        (src.data_ptr(), 16, sink.data_ptr(), W - 1),  # sink too small
    ]
    for args in bad:
        with pytest.raises(ns.NSError):
            ns.ns_read_stream(*args)
