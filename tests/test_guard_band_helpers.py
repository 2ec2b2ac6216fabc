"""The guard-band helpers of test_gpu_guard_bands.py on CPU tensors: a write one
element past either end of the inner view, in any of the buffer types, is reported."""
import pytest
import torch

from test_gpu_guard_bands import GUARD, _guarded, _margins_intact


@pytest.mark.parametrize("dtype", [torch.float32, torch.int32, torch.uint8])
def test_margins_catch_out_of_range_writes(dtype):
    t = torch.zeros((3, 5), dtype=dtype)
    buf, view = _guarded(t)
    assert torch.equal(view, t)
    view.fill_(7)                      # writes inside the view are fine
    _margins_intact(buf, "inside")
    buf[GUARD + t.numel()] = 1         # one past the end
    with pytest.raises(AssertionError, match="past the end"):
        _margins_intact(buf, "after")
    buf2, _ = _guarded(t)
    buf2[GUARD - 1] = 1                # one before the start
    with pytest.raises(AssertionError, match="before the buffer"):
        _margins_intact(buf2, "before")
