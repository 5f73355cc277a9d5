"""pa_read_ceiling (the read-bandwidth calibration) through the C ABI (needs
an MI355X).  It writes nothing unless the bytes it folded equal a fixed
constant, so a buffer holding that constant in one word and zeros elsewhere
shows which tiles were read: the word's tile read once gives the constant,
tiles never read leave the sink at zero, and tile ids outside the buffer
are skipped."""

import pytest
import torch

from helpers import note

pytestmark = pytest.mark.gpu
MAGIC = 0x9E3779B9


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_222_amd as pa
    pa.load()
    return pa


def _buffer(n_tiles, marked_tile, word=100):
    buf = torch.zeros(n_tiles * 1024, dtype=torch.int32)
    buf[marked_tile * 1024 + word] = MAGIC - (1 << 32)   # the same 32 bits
    return buf.cuda()


def _sink():
    return torch.zeros(1, dtype=torch.int32, device="cuda")


def _bits(sink):
    return int(sink.item()) & 0xFFFFFFFF


@pytest.mark.parametrize("n_tiles", [1, 64, 3000])
def test_stream_reads_every_tile(pa, n_tiles):
    buf = _buffer(n_tiles, n_tiles - 1)
    sink = _sink()
    note(f"pa_read_ceiling stream n_tiles={n_tiles}")
    pa.pa_read_ceiling(buf, sink)
    torch.cuda.synchronize()
    assert _bits(sink) == MAGIC


def test_gather_reads_the_named_tiles_only(pa):
    buf = _buffer(64, 63)
    order = torch.tensor([5, 63, -1, 1000, 7], dtype=torch.int32,
                         device="cuda")
    sink = _sink()
    note("pa_read_ceiling gather with out-of-range ids")
    pa.pa_read_ceiling(buf, sink, tile_order=order)
    torch.cuda.synchronize()
    assert _bits(sink) == MAGIC
    sink = _sink()
    order = torch.tensor([5, 62, 0, -7, 64], dtype=torch.int32, device="cuda")
    note("pa_read_ceiling gather without the marked tile")
    pa.pa_read_ceiling(buf, sink, tile_order=order)
    torch.cuda.synchronize()
    assert _bits(sink) == 0


def test_gather_of_many_tiles_in_random_order(pa):
    n = 5000
    buf = _buffer(n, 4321)
    gen = torch.Generator().manual_seed(1)
    order = torch.randperm(n, generator=gen).to(torch.int32).cuda()
    sink = _sink()
    note("pa_read_ceiling gather of a permutation of 5000 tiles")
    pa.pa_read_ceiling(buf, sink, tile_order=order)
    torch.cuda.synchronize()
    assert _bits(sink) == MAGIC


def test_timing_events_bracket_the_read_kernel(pa):
    """pa_time_next_attention also times the next pa_read_ceiling launch:
    its events come back recorded, the interval inside the one measured by
    events around the call, and consumed by that launch."""
    buf = _buffer(20000, 7)
    sink = _sink()
    outer0, outer1, k0, k1 = (torch.cuda.Event(enable_timing=True)
                              for _ in range(4))
    note("pa_read_ceiling with dispatch-timestamp events")
    outer0.record()
    pa.pa_time_next_attention(k0, k1)
    pa.pa_read_ceiling(buf, sink)
    outer1.record()
    torch.cuda.synchronize()
    inner = k0.elapsed_time(k1)
    assert 0.0 < inner <= outer0.elapsed_time(outer1) + 1e-3
    assert _bits(sink) == MAGIC
