"""The streaming-read yardstick (strata_window_stream_read): it reads every word it is
given (the last one included, at ragged sizes), and writes its sink only when the fold
of one lane's words matches the caller's value."""
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import verify_window_expert_amd as sw  # noqa: E402


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 1 << 24, (1 << 24) + 48])
def test_stream_read_folds_every_word(nbytes):
    print(f"[stream] bytes={nbytes}", flush=True)
    src = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    # all-zero words fold to 0 in every thread: magic 0 writes the sink, magic 1 does not
    sink = torch.full((4,), -1, dtype=torch.int32, device="cuda")
    sw.strata_window_stream_read(src, sink, magic=1)
    torch.cuda.synchronize()
    assert sink[0].item() == -1
    sw.strata_window_stream_read(src, sink, magic=0)
    torch.cuda.synchronize()
    assert sink[0].item() == 0
    # one nonzero 16-byte word (the first, one in the middle, the last): only the lane that
    # reads it folds to its value
    words = nbytes // 16
    for w in sorted({0, words // 2, words - 1}):
        src.zero_()
        src[4 * w:4 * w + 4] = torch.tensor([5, 6, 7, 9], dtype=torch.int32, device="cuda")
        sink.fill_(-1)
        sw.strata_window_stream_read(src, sink, magic=5 ^ 6 ^ 7 ^ 9)
        torch.cuda.synchronize()
        assert sink[0].item() == 5 ^ 6 ^ 7 ^ 9, w
