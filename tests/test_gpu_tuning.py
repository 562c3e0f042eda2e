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


@pytest.mark.parametrize("off", [2, 6, 14])
def test_copy_reference_off_the_grid(off):
    """Buffers off the 16-byte grid take unaligned 16-byte accesses: the
    bytes still arrive exactly, and nothing around dst is written."""
    n = 8192 * 5 + 16 * 3
    sbuf = torch.randint(0, 256, (n + 32,), dtype=torch.uint8, device="cuda:0")
    guard = torch.full((n + 512,), 7, dtype=torch.uint8, device="cuda:0")
    src, dst = sbuf[off:off + n], guard[256 + off:256 + off + n]
    tn.copy_reference(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    assert torch.all(guard[:256 + off] == 7) and torch.all(guard[256 + off + n:] == 7)


def test_copy_reference_rejects_bad_arguments():
    a = torch.zeros(4096, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(tn.RMSNormError):
        tn.copy_reference(a[1:4096 - 15], torch.zeros(4080, dtype=torch.uint8, device="cuda:0"))  # odd address
    with pytest.raises(tn.RMSNormError):
        tn.copy_reference(a[:2048], a[1024:3072])  # overlap
    with pytest.raises(ValueError):
        tn.copy_reference(a, a[:16])  # sizes differ
