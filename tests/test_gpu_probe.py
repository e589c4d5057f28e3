"""The measurement aids of include/q8_probe.h on the GPU: the streaming-read probe reads
every word of its buffer exactly once in each launch shape (the xor of its sink equals
the xor of the buffer's 32-bit words), and the empty launch runs."""

from __future__ import annotations

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

q8 = pytest.importorskip("block_quantized_weight_linear_amd")


@pytest.mark.parametrize("chunks", [1, 37, 1024 + 5])
def test_stream_read_reads_every_word_once(chunks):
    dev = torch.device("cuda:0")
    g = torch.Generator().manual_seed(chunks)
    host = torch.randint(0, 256, (chunks * 4096,), dtype=torch.uint8, generator=g)
    buf = host.to(dev)
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    for shape in range(q8.probe_shape_count()):
        sink = q8.probe_stream_read(buf, chunks * 4096, shape)
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        assert got == want, (shape, hex(int(got)), hex(int(want)))


def test_stream_read_rejects_short_buffers_and_bad_shapes():
    dev = torch.device("cuda:0")
    buf = torch.zeros(8192, dtype=torch.uint8, device=dev)
    with pytest.raises(ValueError):
        q8.probe_stream_read(buf, 3 * 4096, 0)
    with pytest.raises(ValueError):
        q8.probe_stream_read(buf, 4096, q8.probe_shape_count())
    with pytest.raises(q8.Q8Error):
        q8.probe_stream_read(buf, 4000, 0)


def test_empty_launch():
    dev = torch.device("cuda:0")
    for blocks in (1, 2048):
        q8.probe_empty(blocks, dev)
    torch.cuda.synchronize()
