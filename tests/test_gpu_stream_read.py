"""GPU: the read-only bandwidth probe (pkv_stream_read) reads every 16-byte
chunk it is given, and only those.

A chunk holding the probe's mark word, in an otherwise zero buffer, makes
the lane that reads it store the mark to the sink; a zero buffer, or a mark
past the requested length, leaves the sink alone.  Buffers span several
passes of the grid (4096 workgroups x 256 lanes x 8 chunks = 128 MiB) and end
in a ragged tail.
"""

import pytest
import torch

from gpu_common import require_gpu

pytestmark = pytest.mark.gpu

MARK = 0x9E3779B9
GRID_CHUNKS = 4096 * 256 * 8


def _run(pkv, nchunks, mark_at=None, nbytes=None):
    buf = torch.zeros(nchunks * 4, dtype=torch.int32, device="cuda")
    if mark_at is not None:
        buf[mark_at * 4] = MARK - (1 << 32)           # the same 32 bits as a signed int32
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    pkv.stream_read(buf, sink, nbytes)
    torch.cuda.synchronize()
    return int(sink.item()) & 0xFFFFFFFF


@pytest.mark.parametrize("nchunks", [1, 1000, GRID_CHUNKS + 3, 2 * GRID_CHUNKS + 1234])
def test_zero_buffer_leaves_the_sink(nchunks):
    pkv = require_gpu()
    print(f"[stream_read] zeros, {nchunks} chunks", flush=True)
    assert _run(pkv, nchunks) == 0


@pytest.mark.parametrize("nchunks,where", [(1, 0), (1000, 999), (GRID_CHUNKS + 3, GRID_CHUNKS + 2),
                                           (2 * GRID_CHUNKS + 1234, 0), (2 * GRID_CHUNKS + 1234, GRID_CHUNKS + 7),
                                           (2 * GRID_CHUNKS + 1234, 2 * GRID_CHUNKS + 1233),
                                           (2 * GRID_CHUNKS + 1234, 512 * 4097 + 64 * 3 + 5)])
def test_every_chunk_is_read(nchunks, where):
    pkv = require_gpu()
    print(f"[stream_read] mark at chunk {where} of {nchunks}", flush=True)
    assert _run(pkv, nchunks, where) == MARK


def test_nothing_past_the_requested_length_is_read():
    pkv = require_gpu()
    n = GRID_CHUNKS + 100
    assert _run(pkv, n, mark_at=n - 1, nbytes=(n - 1) * 16) == 0
    assert _run(pkv, n, mark_at=n - 2, nbytes=(n - 1) * 16) == MARK


def test_binding_checks():
    pkv = require_gpu()
    buf = torch.zeros(64, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        pkv.stream_read(buf, sink, 128)                    # past the buffer
    with pytest.raises(pkv.PagedKVError):
        pkv.stream_read(buf, sink, 24)                     # not whole chunks
    with pytest.raises(ValueError):
        pkv.stream_read(buf.cpu(), sink)
