"""The streaming-read yardstick (strata_window_stream_read): it reads every word it is
given, and writes its sink only when the fold of the words matches the caller's value."""
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
    # one nonzero word (the last): only the thread that reads it folds to its value
    src[-4:] = torch.tensor([5, 6, 7, 9], dtype=torch.int32, device="cuda")
    sink.fill_(-1)
    sw.strata_window_stream_read(src, sink, magic=5 ^ 6 ^ 7 ^ 9)
    torch.cuda.synchronize()
    assert sink[0].item() == 5 ^ 6 ^ 7 ^ 9
