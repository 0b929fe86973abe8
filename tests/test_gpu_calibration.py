"""The calibration read (rimuru_stream_read) visits every 16-byte piece of
its buffer: one planted word whose value is the sink pattern, with zeros
everywhere else, reaches the sink wherever it sits (first piece, middle,
last piece of a ragged size); an all-zero buffer leaves the sink alone."""
import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from paged_moe_expert_amd import rimuru as R

PATTERN = 0x5A5A5A5A


@pytest.mark.parametrize("n_words", [4, 4 * 1000003, 4 * (2048 * 256 * 4 + 7)])
@pytest.mark.parametrize("where", ["first", "middle", "last"])
def test_every_piece_is_read(n_words, where):
    buf = torch.zeros(n_words, dtype=torch.int32, device="cuda")
    pos = {"first": 1, "middle": n_words // 2, "last": n_words - 1}[where]
    buf[pos] = PATTERN
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    R.stream_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink[0].item()) == PATTERN
    buf.zero_()
    sink.zero_()
    R.stream_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink[0].item()) == 0
