"""The streaming-read reference kernel (mtp_stream_read) reads every full 8 KB
unit of its buffer and nothing past them: a 16-byte chunk planted with the
magic value is seen wherever it sits inside the read range (first, middle and
last unit, several grid strides deep) and not when it sits in the tail past
the last full unit."""
import pytest
import torch

from parity import DEV, log, mtp

pytestmark = pytest.mark.gpu

MAGIC = 0x5EED1234


def _seen(nbytes_buf, nbytes_read, offset, shape=0):
    m = mtp()
    buf = torch.zeros(nbytes_buf // 4, dtype=torch.int32, device=DEV)
    buf[offset // 4] = MAGIC  # < 2^31: an int32 as it is
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    m.mtp_stream_read(buf, nbytes_read, MAGIC, sink, shape=shape)
    torch.cuda.synchronize()
    return int(sink.item()) == MAGIC


@pytest.mark.parametrize("shape", [0, 1, 2, 3, 4, 5])
@pytest.mark.parametrize("offset_units", [0, 1, 517, 4095])
def test_planted_chunk_is_read(shape, offset_units):
    n = 4096 * 8192 + 100  # 4096 full 8 KB spans (several grid strides in every shape) and a tail
    off = offset_units * 8192 + 16 * 37
    log(f"stream read: shape {shape}, chunk at {off}")
    assert _seen(n + 12, n, off, shape)


@pytest.mark.parametrize("shape", [0, 1, 2, 3, 4, 5])
def test_tail_past_the_last_unit_is_not_read(shape):
    n = 64 * 8192 + 4096
    assert not _seen(n, n, 64 * 8192 + 16, shape)
    assert _seen(n, n, 63 * 8192 + 8176, shape)
