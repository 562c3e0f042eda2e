"""Property-based checks of the C ABI's argument validation, on the host with
no GPU (hypothesis).  Random sizes, strides, formats, eps values and fake
device addresses: every call returns a status without crashing, arguments
that break a documented rule are rejected (RMSN_ERR_INVALID_ARG or
RMSN_ERR_UNSUPPORTED), and arguments that keep every rule reach the device
query, which fails with RMSN_ERR_HIP because no device is visible (or return
RMSN_OK for an empty batch).  The expected outcome is derived from the rules
the headers state, not from the library's code.

Where a device is visible these tests are skipped: a call that passed
validation would then launch a kernel on the fake addresses.
"""

from __future__ import annotations

import ctypes
import math

import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

from tests.test_abi_cpu import _lib, _no_device_visible  # noqa: E402

pytestmark = pytest.mark.skipif(not _no_device_visible(), reason="runs only where no GPU is visible")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIP = 0, 1, 2, 3, 4
GiB = 1 << 30
# fake device addresses 2^52 bytes apart: no buffer of these tests (< 2^50
# bytes) reaches the next
BASES = [(k + 1) << 52 for k in range(8)]

dtypes = st.sampled_from([0, 1, 2, 3, -1])
eps_values = st.sampled_from([1e-5, 1e-6, 1.0, 0.0, -1e-5, float("nan"), float("inf")])


@settings(max_examples=400, deadline=None)
@given(M=st.integers(-2, 70000), H=st.integers(-2, (1 << 31) + 5), pad=st.integers(-3, 64),
       xdt=dtypes, wdt=dtypes, weighted=st.booleans(), eps=eps_values, with_rrms=st.booleans(),
       misalign=st.booleans())
def test_rmsnorm_fwd_validation(M, H, pad, xdt, wdt, weighted, eps, with_rrms, misalign):
    lib = _lib()
    stride = H + pad
    x, y, w, rr = BASES[0] + (2 if misalign else 0), BASES[1], BASES[2], BASES[3]
    st_ = lib.rmsnorm_fwd(ctypes.c_void_p(x), stride, ctypes.c_void_p(w) if weighted else None, ctypes.c_void_p(y),
                          stride, ctypes.c_void_p(rr) if with_rrms else None, M, H, eps, xdt, wdt, None)
    broken = (xdt not in (0, 1, 2) or (weighted and wdt not in (xdt, 0)) or M < 0 or H < 1 or H > GiB
              or stride < H or not (eps > 0 and math.isfinite(eps)))
    if broken:
        assert st_ in (INVALID, UNSUPPORTED), (st_, lib.rmsnorm_last_error())
        assert lib.rmsnorm_last_error()
    elif M == 0:
        assert st_ == OK
    else:
        assert st_ == HIP, (st_, lib.rmsnorm_last_error())


@settings(max_examples=300, deadline=None)
@given(M=st.integers(1, 5000), H=st.integers(1, 9000), offset_rows=st.integers(-3, 3), offset_elems=st.integers(-40, 40),
       same_stride=st.booleans())
def test_output_may_alias_an_input_only_exactly(M, H, offset_rows, offset_elems, same_stride):
    """y may be x itself (same pointer and stride); any other overlap of
    their byte ranges is rejected."""
    lib = _lib()
    es = 2
    x = BASES[0]
    ystride = H if same_stride else H + 8
    y = x + (offset_rows * H + offset_elems) * es
    st_ = lib.rmsnorm_fwd(ctypes.c_void_p(x), H, None, ctypes.c_void_p(y), ystride, None, M, H, 1e-5, 2, 2, None)
    x_lo, x_hi = x, x + M * H * es
    y_lo, y_hi = y, y + ((M - 1) * ystride + H) * es
    overlap = x_lo < y_hi and y_lo < x_hi
    same = y == x and ystride == H
    if overlap and not same:
        assert st_ == INVALID, lib.rmsnorm_last_error()
    else:
        assert st_ == HIP, (st_, lib.rmsnorm_last_error())


@settings(max_examples=300, deadline=None)
@given(M=st.integers(-1, 5000), H=st.integers(1, 20000), ws_delta=st.integers(-64, 64), want_dw=st.booleans(),
       weighted=st.booleans(), ws_misalign=st.booleans(), with_dres=st.booleans())
def test_backward_workspace_rules(M, H, ws_delta, want_dw, weighted, ws_misalign, with_dres):
    lib = _lib()
    need = lib.rmsnorm_bwd_workspace_bytes(M, H)
    assert need == (0 if M <= 0 else min(M, min(max((8 << 20) // (4 * H), 1024), 8192)) * H * 4)
    ws_bytes = max(0, need + ws_delta)
    ws = BASES[6] + (8 if ws_misalign else 0)
    args = [ctypes.c_void_p(BASES[0]), H, ctypes.c_void_p(BASES[1]), H]
    tail = [ctypes.c_void_p(BASES[2]) if weighted else None, ctypes.c_void_p(BASES[3]), ctypes.c_void_p(BASES[4]), H,
            ctypes.c_void_p(BASES[5]) if want_dw else None, ctypes.c_void_p(ws), ws_bytes, M, H, 2, 2, None]
    if with_dres:
        st_ = lib.rmsnorm_bwd_residual(*args, ctypes.c_void_p(BASES[7]), H, *tail)
    else:
        st_ = lib.rmsnorm_bwd(*args, *tail)
    if M < 0 or (want_dw and not weighted):
        assert st_ == INVALID, lib.rmsnorm_last_error()
    elif want_dw and M > 0 and (ws_bytes < need or ws_misalign):
        assert st_ == WORKSPACE, lib.rmsnorm_last_error()
    elif M == 0 and not want_dw:
        assert st_ == OK
    else:
        # a valid call (including dw of zero rows, which writes zeros) needs the device
        assert st_ == HIP, (st_, lib.rmsnorm_last_error())


@settings(max_examples=400, deadline=None)
@given(B=st.integers(-1, 4), S=st.integers(-1, 50), NH=st.integers(-1, 40), D=st.integers(-2, 300),
       head_pad=st.integers(-4, 16), row_pad=st.integers(-70, 64), table_cols=st.integers(0, 300),
       xdt=dtypes, tdt=dtypes, in_place=st.booleans())
def test_rope_validation(B, S, NH, D, head_pad, row_pad, table_cols, xdt, tdt, in_place):
    lib = _lib()
    hs = D + head_pad
    rs = max(NH, 1) * max(hs, 0) + row_pad
    x = BASES[0]
    out = x if in_place else BASES[1]
    st_ = lib.rope_apply(ctypes.c_void_p(x), rs, hs, ctypes.c_void_p(BASES[2]), ctypes.c_void_p(BASES[3]), table_cols,
                         ctypes.c_void_p(out), rs, hs, B, S, NH, D, 0, xdt, tdt, None)
    broken = (xdt not in (0, 1, 2) or tdt not in (xdt, 0) or B < 0 or S < 1 or NH < 1 or D < 2 or D % 2
              or hs < D or rs < (NH - 1) * hs + D or table_cols < D // 2)
    if broken:
        assert st_ in (INVALID, UNSUPPORTED), (st_, lib.rmsnorm_last_error())
    elif B == 0:
        assert st_ == OK
    else:
        assert st_ == HIP, (st_, lib.rmsnorm_last_error())


@settings(max_examples=200, deadline=None)
@given(M=st.integers(-1, 3000), H=st.integers(-1, 5000), wdt=dtypes, weighted=st.booleans(), biased=st.booleans(),
       eps=eps_values, resid=st.booleans())
def test_layernorm_validation(M, H, wdt, weighted, biased, eps, resid):
    lib = _lib()
    xdt = 2
    w = ctypes.c_void_p(BASES[2]) if weighted else None
    b = ctypes.c_void_p(BASES[3]) if biased else None
    if resid:
        st_ = lib.layernorm_fwd_residual(ctypes.c_void_p(BASES[0]), max(H, 1), ctypes.c_void_p(BASES[4]), max(H, 1), w,
                                         b, ctypes.c_void_p(BASES[1]), max(H, 1), ctypes.c_void_p(BASES[5]), max(H, 1),
                                         None, None, M, H, eps, xdt, wdt, None)
    else:
        st_ = lib.layernorm_fwd(ctypes.c_void_p(BASES[0]), max(H, 1), w, b, ctypes.c_void_p(BASES[1]), max(H, 1),
                                None, None, M, H, eps, xdt, wdt, None)
    broken = ((weighted or biased) and wdt not in (xdt, 0)) or M < 0 or H < 1 or not (eps > 0 and math.isfinite(eps))
    if broken:
        assert st_ in (INVALID, UNSUPPORTED), (st_, lib.rmsnorm_last_error())
    elif M == 0:
        assert st_ == OK
    else:
        assert st_ == HIP, (st_, lib.rmsnorm_last_error())
