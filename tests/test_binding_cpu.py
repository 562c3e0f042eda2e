"""Host logic of the Python binding, on the CPU: how a tensor is viewed as
rows (count, length and one row stride in elements) before its pointer and
strides are handed to the C ABI.  CPU tensors stand in for device tensors
(the view logic reads only shapes and strides; nothing is launched)."""

from __future__ import annotations

import pytest

torch = pytest.importorskip("torch")

import transformer_normalization_amd as tn  # noqa: E402


class DeviceView:
    """A CPU tensor that reports itself as a device tensor and as
    non-contiguous, so that _rows takes its general stride path."""

    is_cuda = True

    def __init__(self, t):
        self.t = t

    def is_contiguous(self):
        return False

    def dim(self):
        return self.t.dim()

    def stride(self, d):
        return self.t.stride(d)

    def numel(self):
        return self.t.numel()

    @property
    def shape(self):
        return self.t.shape


def rows(t):
    return tn._rows(DeviceView(t), "t")


def test_plain_and_padded_rows():
    assert rows(torch.zeros(5, 7)) == (5, 7, 7)
    assert rows(torch.zeros(5, 12)[:, :7]) == (5, 7, 12)
    assert rows(torch.zeros(2, 3, 19)[..., :7]) == (6, 7, 19)


def test_size_one_dims_carry_no_stride():
    """A [B, 1, H] per-batch slice of a modulation tensor: torch gives the
    size-1 dim a stride of its own choosing (H after unsqueeze); the rows are
    B apart by the modulation tensor's row stride."""
    mod = torch.zeros(3, 2 * 7 + 5)
    assert rows(mod[:, :7].unsqueeze(1)) == (3, 7, 19)
    assert rows(mod.view(3, 1, 19)[..., 7:14]) == (3, 7, 19)
    assert rows(torch.zeros(1, 1, 12)[..., :7]) == (1, 7, 7)
    assert rows(torch.zeros(4, 1, 3, 19)[..., :7]) == (12, 7, 19)


def test_uniformly_strided_leading_dims_collapse():
    # rows a * 114 + b * 38 = (3 a + b) * 38: one stride of 38
    assert rows(torch.zeros(4, 6, 19)[:, ::2, :7]) == (12, 7, 38)


def test_leading_dims_without_one_stride_are_rejected():
    with pytest.raises(ValueError, match="one stride"):
        rows(torch.zeros(4, 6, 19)[:, :3, :7])  # rows 19 apart inside a block, 114 between blocks


def test_last_dim_must_be_contiguous():
    with pytest.raises(ValueError, match="contiguous along its last dimension"):
        rows(torch.zeros(5, 14)[:, ::2])
