"""Host-side checks of the Python binding (no GPU): caller-supplied outputs
must have exactly the dtype, shape and device a call writes."""
import pytest
import torch

from moe_variable_size_amd.api import _require_out


def test_output_of_the_exact_shape_passes():
    _require_out(torch.empty(4, 6), "y", torch.float32, (4, 6), "cpu")


@pytest.mark.parametrize("t,exc", [
    (torch.empty(4, 5), ValueError),                      # too few columns: would be written past
    (torch.empty(3, 6), ValueError),                      # too few rows
    (torch.empty(24), ValueError),                        # right size, wrong shape
    (torch.empty(4, 6, dtype=torch.float64), TypeError),  # wrong dtype
    (torch.empty(6, 4).t(), ValueError),                  # not contiguous
    ([0.0] * 24, TypeError),                              # not a tensor
])
def test_bad_outputs_are_rejected(t, exc):
    with pytest.raises(exc):
        _require_out(t, "y", torch.float32, (4, 6), "cpu")


def test_output_on_another_device_is_rejected():
    with pytest.raises(ValueError):
        _require_out(torch.empty(4, 6), "y", torch.float32, (4, 6), "meta")
