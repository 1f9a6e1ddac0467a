"""q8_stream_read, the streaming-read ceiling kernel: every byte of the buffer
is read exactly once, checked through the XOR checksum it leaves in the sink
(compared with numpy's XOR of the same 32-bit words) for sizes below one wave's
access, ragged against the grid, and larger than the grid's first pass."""
import numpy as np
import pytest
import torch

from decode_q8_amd import q8
from tests.gpu_helpers import dev, down, require_gpu, up

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _words(nbytes, seed):
    return np.random.default_rng(seed).integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)


@pytest.mark.parametrize("nbytes", [16, 1024 + 16, 256 * 16 * 3 + 48, (4 << 20) + 16 * 7, 96 << 20])
def test_reads_every_word_once(nbytes):
    w = _words(nbytes, nbytes)
    buf = up(w.view(np.int32))
    sink = torch.zeros(4, dtype=torch.int32, device=dev())
    q8.q8_stream_read(buf, nbytes, sink)
    got = int(down(sink)[0]) & 0xFFFFFFFF
    assert got == int(np.bitwise_xor.reduce(w)), nbytes
    assert not down(sink)[1:].any()  # nothing written past the sink word


def test_xors_into_the_sink_and_repeats():
    nbytes = (1 << 20) + 32
    w = _words(nbytes, 7)
    buf = up(w.view(np.int32))
    start = np.array([0x5A5A1234], dtype=np.uint32)
    sink = up(start.view(np.int32))
    q8.q8_stream_read(buf, nbytes, sink)
    assert int(down(sink)[0]) & 0xFFFFFFFF == int(start[0] ^ np.bitwise_xor.reduce(w))
    q8.q8_stream_read(buf, nbytes, sink)  # a second pass cancels the first
    assert int(down(sink)[0]) & 0xFFFFFFFF == int(start[0])
