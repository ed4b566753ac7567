"""GPU checks of the read-bandwidth probe tq_stream_read: it reads every
16-byte chunk of its buffer (a marker word planted anywhere reaches the sink),
writes nothing else, and rejects bad arguments."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_vector_02_amd as lib
    return lib


MARK = 0x9E3779B9 - (1 << 32)  # the probe's marker as a signed int32


@pytest.mark.parametrize("n_words,where", [(4, 0), (1 << 20, 123457), (1 << 20, (1 << 20) - 1),
                                           ((1 << 22) + 12, (1 << 22) + 9), (64 * 1024 * 1024, 5_000_001)])
def test_every_chunk_is_read(tq, n_words, where):
    src = torch.zeros(n_words, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    tq.tq_stream_read(src, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0  # an all-zero buffer never matches the marker
    src[where] = MARK  # the lane that reads this chunk ends with the marker alone
    tq.tq_stream_read(src, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == MARK


def test_bad_arguments(tq):
    src = torch.zeros(6, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(tq.TQError):
        tq.tq_stream_read(src, sink)  # 24 bytes: not a multiple of 16
    with pytest.raises(tq.TQError):
        tq.tq_stream_read(src[1:5], sink)  # not 16-byte aligned
