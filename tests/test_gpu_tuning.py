"""The development hooks of include/rmsnorm_tuning.h on the GPU: the
speed-of-light copy moves the bytes exactly and refuses bad arguments."""

from __future__ import annotations

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import transformer_normalization_amd as tn  # noqa: E402


@pytest.mark.parametrize("nbytes", [16, 4096, 8192, 8192 * 7 + 16 * 3, 64 << 20])
def test_copy_reference_copies_exactly(nbytes):
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda:0")
    guard = torch.full((nbytes + 512,), 7, dtype=torch.uint8, device="cuda:0")
    dst = guard[256:256 + nbytes]
    tn.copy_reference(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    assert torch.all(guard[:256] == 7) and torch.all(guard[256 + nbytes:] == 7)


def test_copy_reference_rejects_bad_arguments():
    a = torch.zeros(4096, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(tn.RMSNormError):
        tn.copy_reference(a[8:4096 - 8], torch.zeros(4080, dtype=torch.uint8, device="cuda:0"))  # misaligned
    with pytest.raises(tn.RMSNormError):
        tn.copy_reference(a[:2048], a[1024:3072])  # overlap
    with pytest.raises(ValueError):
        tn.copy_reference(a, a[:16])  # sizes differ
