"""rmsnorm_bwd_noalloc: the backward whose dw partial rows live in the
library's static device scratch, for callers that cannot allocate.  Its
outputs must equal rmsnorm_bwd's bit for bit (same kernels, same partial-row
count), over consecutive calls that reuse the scratch, the second smaller
than the first, and a call too large for the scratch is rejected before
anything is enqueued."""

from __future__ import annotations

import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synthetic  # noqa: E402
import transformer_normalization_amd as tn  # noqa: E402
from tests import gpu_util as G  # noqa: E402

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs an MI355X", allow_module_level=True)


def _case(seed, M, H):
    x = synthetic.normal_tensor(seed, synthetic.STREAM_X, (M, H), "bf16")
    dy = synthetic.normal_tensor(seed, synthetic.STREAM_DY, (M, H), "bf16")
    w = synthetic.normal_tensor(seed, synthetic.STREAM_W, (H,), "bf16", 1.0, 0.1)
    xd, dyd, wd = G.to_dev(x, "bf16"), G.to_dev(dy, "bf16"), G.to_dev(w, "bf16")
    _, rr = tn.rmsnorm_fwd(xd, wd, 1e-6, return_rrms=True)
    return dyd, xd, wd, rr.reshape(-1).contiguous()


def _noalloc(dy, x, w, rr):
    """One call through the C ABI, outputs preallocated."""
    lib = tn.load_library()
    M, H = x.shape
    dx = torch.full_like(x, float("nan"))
    dw = None if w is None else torch.full((H,), float("nan"), dtype=torch.float32, device=x.device)
    st = lib.rmsnorm_bwd_noalloc(dy.data_ptr(), H, x.data_ptr(), H, None if w is None else w.data_ptr(),
                                 rr.data_ptr(), dx.data_ptr(), H, None if dw is None else dw.data_ptr(), M, H,
                                 tn.RMSN_BF16, tn.RMSN_BF16, torch.cuda.current_stream().cuda_stream)
    assert st == 0, tn.load_library().rmsnorm_last_error().decode()
    return dx, dw


def test_noalloc_matches_workspace_backward_over_consecutive_calls():
    # first the bf16 8192 x 6144 backward (6 MiB of partial rows), then a
    # smaller call off the 16-byte grid that reuses the same scratch
    for seed, M, H in ((1201, 8192, 6144), (1202, 257, 4097)):
        print(f"[gpu] noalloc M={M} H={H}", flush=True)
        dy, x, w, rr = _case(seed, M, H)
        ref_dx, ref_dw = tn.rmsnorm_bwd(dy, x, w, rr)
        dx, dw = _noalloc(dy, x, w, rr)
        torch.cuda.synchronize()
        assert torch.equal(dx.view(torch.int16), ref_dx.view(torch.int16)), (M, H)
        assert torch.equal(dw.view(torch.int32), ref_dw.view(torch.int32)), (M, H)


def test_noalloc_long_rows_off_the_grid_reuse_the_scratch():
    # rows off the grid longer than one tile take two passes; beyond 65536
    # columns their later chunks zero and then add into the workgroup's
    # partial row at every row, here in the static scratch, so a second call
    # with other data must not see the first one's sums; then a shorter row
    for seed, M, H in ((1203, 32, 70001), (1204, 32, 70001), (1205, 24, 30001)):
        print(f"[gpu] noalloc M={M} H={H}", flush=True)
        dy, x, w, rr = _case(seed, M, H)
        ref_dx, ref_dw = tn.rmsnorm_bwd(dy, x, w, rr)
        dx, dw = _noalloc(dy, x, w, rr)
        torch.cuda.synchronize()
        assert torch.equal(dx.view(torch.int16), ref_dx.view(torch.int16)), (M, H)
        assert torch.equal(dw.view(torch.int32), ref_dw.view(torch.int32)), (M, H)


def test_noalloc_weightless_and_binding():
    dy, x, _, rr = _case(1203, 64, 1000)
    ref_dx, _ = tn.rmsnorm_bwd(dy, x, None, rr)
    dx = torch.empty_like(x)
    got, dw = tn.rmsnorm_bwd_noalloc(dy, x, None, rr, dx)
    torch.cuda.synchronize()
    assert dw is None and got.data_ptr() == dx.data_ptr()
    assert torch.equal(dx.view(torch.int16), ref_dx.view(torch.int16))


def test_noalloc_rejects_calls_beyond_the_scratch():
    # bf16 rows of 65536 take 256 partial rows of 256 KiB: 64 MiB > 32 MiB
    M, H = 512, 65536
    x = torch.zeros((M, H), dtype=torch.bfloat16, device=G.DEV)
    w = torch.ones(H, dtype=torch.bfloat16, device=G.DEV)
    rr = torch.ones(M, dtype=torch.float32, device=G.DEV)
    dx = torch.full_like(x, 7.0)
    dw = torch.full((H,), 7.0, dtype=torch.float32, device=G.DEV)
    lib = tn.load_library()
    st = lib.rmsnorm_bwd_noalloc(x.data_ptr(), H, x.data_ptr(), H, w.data_ptr(), rr.data_ptr(), dx.data_ptr(), H,
                                 dw.data_ptr(), M, H, tn.RMSN_BF16, tn.RMSN_BF16, torch.cuda.current_stream().cuda_stream)
    assert st == 3, st  # RMSN_ERR_WORKSPACE
    assert b"static scratch" in lib.rmsnorm_last_error()
    torch.cuda.synchronize()
    assert bool((dx == 7.0).all()) and bool((dw == 7.0).all())
    # without dw the scratch is not needed
    st = lib.rmsnorm_bwd_noalloc(x.data_ptr(), H, x.data_ptr(), H, w.data_ptr(), rr.data_ptr(), dx.data_ptr(), H,
                                 None, M, H, tn.RMSN_BF16, tn.RMSN_BF16, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert bool((dx == 0).all())
