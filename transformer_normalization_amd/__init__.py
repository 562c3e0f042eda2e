"""RMSNorm for AMD Instinct MI355X (gfx950): thin Python binding of librmsnorm.so.

The functions below only marshal torch tensors into the C ABI declared in
include/rmsnorm.h (device pointers, row strides in elements, dtype codes and
the current HIP stream); every step of the computation runs in the library's
HIP kernels.  There is no CPU fallback: without the built library the
functions raise.

    y = rmsnorm_fwd(x, w, eps)                       # w may be None
    y, rrms = rmsnorm_fwd(x, w, eps, return_rrms=True)
    y, res_out = rmsnorm_fwd_residual(x, residual, w, eps)
    y = rmsnorm_adaln_fwd(x, w, scale, shift, eps)  # scale/shift [B,S,H] or [B,1,H]
    dx, dw = rmsnorm_bwd(dy, x, w, rrms)
    dh, dw = rmsnorm_bwd_residual(dy, res_out, dres, w, rrms)  # grad of x and residual
    q = rope_apply(q, cos, sin)                      # q [B, S, heads, head_dim], cos/sin [S, head_dim]
    y, h = layernorm_fwd_residual(x, residual, w, b, eps)   # residual + LayerNorm

transformer_normalization_amd.autograd wraps these as torch.autograd
Functions and nn.Modules for training.
"""

from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "librmsnorm.so")

RMSN_F32, RMSN_F16, RMSN_BF16 = 0, 1, 2
STATUS = {0: "RMSN_OK", 1: "RMSN_ERR_INVALID_ARG", 2: "RMSN_ERR_UNSUPPORTED", 3: "RMSN_ERR_WORKSPACE",
          4: "RMSN_ERR_HIP"}
EXPORTED = ("rmsnorm_fwd", "rmsnorm_fwd_residual", "rmsnorm_adaln_fwd", "rmsnorm_bwd_workspace_bytes",
            "rmsnorm_bwd", "rmsnorm_bwd_residual", "rmsnorm_status_string", "rmsnorm_last_error", "rope_apply",
            "layernorm_fwd", "layernorm_fwd_residual")

_lock = threading.Lock()
_lib = None


class RMSNormError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load librmsnorm.so (raises if it has not been built)."""
    global _lib
    lib = _lib
    if lib is not None and path == LIB_PATH:  # loaded: no lock on the per-call path
        return lib
    with _lock:
        if _lib is not None and path == LIB_PATH:
            return _lib
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with `python -m transformer_normalization_amd.build`")
        lib = ctypes.CDLL(path)
        vp, i64, f32, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_size_t
        lib.rmsnorm_fwd.argtypes = [vp, i64, vp, vp, i64, vp, i64, i64, f32, i32, i32, vp]
        lib.rmsnorm_fwd.restype = i32
        lib.rmsnorm_fwd_residual.argtypes = [vp, i64, vp, i64, vp, vp, i64, vp, i64, vp, i64, i64, f32, i32, i32, vp]
        lib.rmsnorm_fwd_residual.restype = i32
        lib.rmsnorm_adaln_fwd.argtypes = [vp, i64, vp, vp, vp, i64, i64, vp, i64, vp, i64, i64, f32, i32, i32, vp]
        lib.rmsnorm_adaln_fwd.restype = i32
        lib.rmsnorm_bwd_workspace_bytes.argtypes = [i64, i64]
        lib.rmsnorm_bwd_workspace_bytes.restype = sz
        lib.rmsnorm_bwd.argtypes = [vp, i64, vp, i64, vp, vp, vp, i64, vp, vp, sz, i64, i64, i32, i32, vp]
        lib.layernorm_fwd.restype = i32
        lib.layernorm_fwd.argtypes = [vp, i64, vp, vp, vp, i64, vp, vp, i64, i64, f32, i32, i32, vp]
        lib.layernorm_fwd_residual.restype = i32
        lib.layernorm_fwd_residual.argtypes = [vp, i64, vp, i64, vp, vp, vp, i64, vp, i64, vp, vp, i64, i64, f32, i32,
                                               i32, vp]
        lib.rmsnorm_tuning_copy.restype = i32
        lib.rmsnorm_tuning_copy.argtypes = [vp, vp, i64, vp]
        lib.rope_apply.restype = i32
        lib.rope_apply.argtypes = [vp, i64, i64, vp, vp, i64, vp, i64, i64, i64, i64, i64, i64, i32, i32, i32, vp]
        lib.rmsnorm_bwd_residual.restype = i32
        lib.rmsnorm_bwd_residual.argtypes = [vp, i64, vp, i64, vp, i64, vp, vp, vp, i64, vp, vp, sz, i64, i64, i32,
                                             i32, vp]
        lib.rmsnorm_bwd.restype = i32
        lib.rmsnorm_bwd_noalloc.argtypes = [vp, i64, vp, i64, vp, vp, vp, i64, vp, i64, i64, i32, i32, vp]
        lib.rmsnorm_bwd_noalloc.restype = i32
        lib.rmsnorm_status_string.argtypes = [i32]
        lib.rmsnorm_status_string.restype = ctypes.c_char_p
        lib.rmsnorm_last_error.argtypes = []
        lib.rmsnorm_last_error.restype = ctypes.c_char_p
        lib.rmsnorm_tuning_set_geometry.argtypes = [i32, i32, i32, i32, i64]
        lib.rmsnorm_tuning_set_geometry.restype = None
        lib.rmsnorm_tuning_set_streaming.argtypes = [i32]
        lib.rmsnorm_tuning_set_streaming.restype = None
        lib.rmsnorm_tuning_tile.argtypes = [i32, i64, i32, i32, ctypes.POINTER(ctypes.c_int32)]
        lib.rmsnorm_tuning_tile.restype = i32
        if path == LIB_PATH:
            _lib = lib
        return lib


def _check(lib, status: int):
    if status != 0:
        raise RMSNormError(status, lib.rmsnorm_last_error().decode())


def _torch():
    import torch
    return torch


_CODES = None


def _dtype_code(t) -> int:
    global _CODES
    if _CODES is None:
        torch = _torch()
        _CODES = {torch.float32: RMSN_F32, torch.float16: RMSN_F16, torch.bfloat16: RMSN_BF16}
    code = _CODES.get(t.dtype)
    if code is None:
        raise TypeError(f"unsupported dtype {t.dtype}; expected float32, float16 or bfloat16")
    return code


def _rows(t, name):
    """(M, H, row stride) of a tensor viewed as rows over its last dim."""
    if t.is_cuda and t.is_contiguous() and t.dim() >= 1:  # the common case, in a few calls
        H = t.shape[-1]
        n = t.numel()
        return (n // H if H else 0), H, max(H, 1)
    if t.dim() < 1:
        raise ValueError(f"{name} must have at least one dimension")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    H = t.shape[-1]
    if t.numel() == 0:
        return 0, H, max(H, 1)
    if t.stride(-1) != 1 and H > 1:
        raise ValueError(f"{name} must be contiguous along its last dimension")
    if t.dim() == 1:
        return 1, H, H
    # leading dims of size > 1 must collapse into one row stride; a dim of
    # size 1 has no meaningful stride (torch gives it any value) and is skipped
    lead = [d for d in range(t.dim() - 1) if t.shape[d] != 1]
    if not lead:
        return 1, H, H
    stride = t.stride(lead[-1])
    expect = stride
    for d in reversed(lead):
        if t.stride(d) != expect:
            raise ValueError(f"{name}'s leading dimensions cannot be viewed as rows with one stride")
        expect *= t.shape[d]
    M = 1
    for d in lead:
        M *= t.shape[d]
    return M, H, stride


def _stream(t):
    """The raw handle of the current HIP stream of t's device."""
    torch = _torch()
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:  # the handle without building a Stream object
        return ctypes.c_void_p(raw(t.device.index if t.device.index is not None else torch.cuda.current_device()))
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def rmsnorm_fwd(x, weight=None, eps: float = 1e-6, out=None, rrms=None, return_rrms: bool = False):
    """y = x * rsqrt(mean(x^2, -1) + eps) * weight over the last dim of x.

    out (same shape and dtype as x, may be x itself) and rrms (float32, one
    value per row) are optional preallocated outputs."""
    torch = _torch()
    lib = load_library()
    M, H, xs = _rows(x, "x")
    if out is None:
        out = torch.empty_like(x, memory_format=torch.contiguous_format)
    if out.shape != x.shape or out.dtype != x.dtype:
        raise ValueError("out must match x in shape and dtype")
    _, _, ys = _rows(out, "out")
    if return_rrms and rrms is None:
        rrms = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    if rrms is not None and (rrms.dtype != torch.float32 or rrms.numel() != M or not rrms.is_contiguous()):
        raise ValueError("rrms must be a contiguous float32 tensor with one value per row")
    wcode = _dtype_code(weight) if weight is not None else _dtype_code(x)
    if weight is not None and (weight.numel() != H or not weight.is_contiguous()):
        raise ValueError("weight must be a contiguous tensor of H elements")
    st = lib.rmsnorm_fwd(_ptr(x), xs, _ptr(weight), _ptr(out), ys, _ptr(rrms), M, H, float(eps), _dtype_code(x),
                         wcode, _stream(x))
    _check(lib, st)
    return (out, rrms) if return_rrms else out


def rmsnorm_fwd_residual(x, residual, weight=None, eps: float = 1e-6, out=None, residual_out=None, rrms=None,
                         return_rrms: bool = False, write_residual: bool = True):
    """h = x + residual (float32), residual_out = h in x's dtype, y = RMSNorm(h).

    Returns (y, residual_out) (plus rrms when return_rrms).  residual_out may
    be `residual` itself for an in-place update of the residual stream."""
    torch = _torch()
    lib = load_library()
    M, H, xs = _rows(x, "x")
    if residual.shape != x.shape or residual.dtype != x.dtype:
        raise ValueError("residual must match x in shape and dtype")
    _, _, rs = _rows(residual, "residual")
    if out is None:
        out = torch.empty_like(x, memory_format=torch.contiguous_format)
    _, _, ys = _rows(out, "out")
    if write_residual and residual_out is None:
        residual_out = torch.empty_like(x, memory_format=torch.contiguous_format)
    ros = 0
    if residual_out is not None:
        if residual_out.shape != x.shape or residual_out.dtype != x.dtype:
            raise ValueError("residual_out must match x in shape and dtype")
        _, _, ros = _rows(residual_out, "residual_out")
    if return_rrms and rrms is None:
        rrms = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    if rrms is not None and (rrms.dtype != torch.float32 or rrms.numel() != M or not rrms.is_contiguous()):
        raise ValueError("rrms must be a contiguous float32 tensor with one value per row")
    wcode = _dtype_code(weight) if weight is not None else _dtype_code(x)
    if weight is not None and (weight.numel() != H or not weight.is_contiguous()):
        raise ValueError("weight must be a contiguous tensor of H elements")
    st = lib.rmsnorm_fwd_residual(_ptr(x), xs, _ptr(residual), rs, _ptr(weight), _ptr(out), ys, _ptr(residual_out),
                                  ros, _ptr(rrms), M, H, float(eps), _dtype_code(x), wcode, _stream(x))
    _check(lib, st)
    res = (out, residual_out)
    return res + (rrms,) if return_rrms else res


def rmsnorm_adaln_fwd(x, weight, scale, shift, eps: float = 1e-6, out=None, rrms=None, return_rrms: bool = False):
    """AdaLN-RMSNorm: (x * rrms) * weight * (1 + scale) + shift over the last dim.

    x is (..., S, H) or (M, H).  scale and shift are either per row (same
    leading shape as x, or (M, H)) or per batch ((B, 1, H) for x of shape
    (B, S, H)); they must share one format (x's or float32, the weight's too)
    and one row stride, as slices of one modulation tensor do."""
    torch = _torch()
    lib = load_library()
    M, H, xs = _rows(x, "x")
    if scale.shape != shift.shape:
        raise ValueError("scale and shift must have the same shape")
    if scale.dtype != shift.dtype:
        raise ValueError("scale and shift must have the same dtype")
    if scale.shape[-1] != H:
        raise ValueError("scale/shift last dim must be H")
    if scale.numel() == M * H or (M == 0 and scale.numel() == 0):
        rows_per_cond = 1
    elif x.dim() >= 2 and scale.dim() == x.dim() and scale.shape[-2] == 1 and \
            tuple(scale.shape[:-2]) == tuple(x.shape[:-2]):
        rows_per_cond = x.shape[-2]
    else:
        raise ValueError("scale/shift must be per row (shape of x) or per batch ([..., 1, H])")
    C, _, cs = _rows(scale, "scale")
    _, _, hs = _rows(shift, "shift")
    if C > 1 and cs != hs:
        raise ValueError("scale and shift must have the same row stride")
    if out is None:
        out = torch.empty_like(x, memory_format=torch.contiguous_format)
    _, _, ys = _rows(out, "out")
    if return_rrms and rrms is None:
        rrms = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    if rrms is not None and (rrms.dtype != torch.float32 or rrms.numel() != M or not rrms.is_contiguous()):
        raise ValueError("rrms must be a contiguous float32 tensor with one value per row")
    pcode = _dtype_code(scale)
    if weight is not None:
        if weight.numel() != H or not weight.is_contiguous():
            raise ValueError("weight must be a contiguous tensor of H elements")
        if weight.dtype != scale.dtype:
            raise ValueError("weight, scale and shift must share one dtype")
    st = lib.rmsnorm_adaln_fwd(_ptr(x), xs, _ptr(weight), _ptr(scale), _ptr(shift), cs, rows_per_cond, _ptr(out),
                               ys, _ptr(rrms), M, H, float(eps), _dtype_code(x), pcode, _stream(x))
    _check(lib, st)
    return (out, rrms) if return_rrms else out


def rmsnorm_bwd_workspace_bytes(M: int, H: int) -> int:
    return int(load_library().rmsnorm_bwd_workspace_bytes(M, H))


def _bwd(dy, x, dres, weight, rrms, dx, dw, workspace, want_dw):
    torch = _torch()
    lib = load_library()
    M, H, xs = _rows(x, "x")
    if dy.shape != x.shape or dy.dtype != x.dtype:
        raise ValueError("dy must match x in shape and dtype")
    _, _, dys = _rows(dy, "dy")
    drs = 0
    if dres is not None:
        if dres.shape != x.shape or dres.dtype != x.dtype:
            raise ValueError("dres must match x in shape and dtype")
        _, _, drs = _rows(dres, "dres")
    if dx is None:
        dx = torch.empty_like(x, memory_format=torch.contiguous_format)
    if dx.shape != x.shape or dx.dtype != x.dtype:
        raise ValueError("dx must match x in shape and dtype")
    _, _, dxs = _rows(dx, "dx")
    if rrms.dtype != torch.float32 or rrms.numel() != M or not rrms.is_contiguous():
        raise ValueError("rrms must be a contiguous float32 tensor with one value per row")
    if weight is not None and (weight.numel() != H or not weight.is_contiguous()):
        raise ValueError("weight must be a contiguous tensor of H elements")
    if weight is not None and want_dw and dw is None:
        dw = torch.empty(H, dtype=torch.float32, device=x.device)
    if weight is None:
        dw = None
    ws_bytes = 0
    if dw is not None:
        need = int(lib.rmsnorm_bwd_workspace_bytes(M, H))
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
        ws_bytes = workspace.numel() * workspace.element_size()
    wcode = _dtype_code(weight) if weight is not None else _dtype_code(x)
    if dres is None:
        st = lib.rmsnorm_bwd(_ptr(dy), dys, _ptr(x), xs, _ptr(weight), _ptr(rrms), _ptr(dx), dxs, _ptr(dw),
                             _ptr(workspace), ws_bytes, M, H, _dtype_code(x), wcode, _stream(x))
    else:
        st = lib.rmsnorm_bwd_residual(_ptr(dy), dys, _ptr(x), xs, _ptr(dres), drs, _ptr(weight), _ptr(rrms),
                                      _ptr(dx), dxs, _ptr(dw), _ptr(workspace), ws_bytes, M, H, _dtype_code(x), wcode,
                                      _stream(x))
    _check(lib, st)
    return dx, dw


def rmsnorm_bwd(dy, x, weight, rrms, dx=None, dw=None, workspace=None, want_dw: bool = True):
    """Gradients of RMSNorm from the saved per-row rrms.

    Returns (dx, dw); dw (float32, shape (H,)) is None for a weightless norm
    or when want_dw is False.  dx may be dy or x itself."""
    return _bwd(dy, x, None, weight, rrms, dx, dw, workspace, want_dw)


def rmsnorm_bwd_noalloc(dy, x, weight, rrms, dx, dw=None):
    """rmsnorm_bwd for callers that cannot allocate (HIP graph capture,
    serving loops): dx (and dw, float32 (H,), when weight is given) must be
    passed in; the dw partial rows go to the library's static device scratch
    (include/rmsnorm.h).  Calls that overlap in time on one device race on
    that scratch.  Returns (dx, dw)."""
    torch = _torch()
    lib = load_library()
    M, H, xs = _rows(x, "x")
    if dy.shape != x.shape or dy.dtype != x.dtype:
        raise ValueError("dy must match x in shape and dtype")
    _, _, dys = _rows(dy, "dy")
    if dx is None or dx.shape != x.shape or dx.dtype != x.dtype:
        raise ValueError("dx must be given, matching x in shape and dtype")
    _, _, dxs = _rows(dx, "dx")
    if rrms.dtype != torch.float32 or rrms.numel() != M or not rrms.is_contiguous():
        raise ValueError("rrms must be a contiguous float32 tensor with one value per row")
    if weight is not None and (weight.numel() != H or not weight.is_contiguous()):
        raise ValueError("weight must be a contiguous tensor of H elements")
    if weight is None:
        dw = None
    elif dw is not None and (dw.dtype != torch.float32 or dw.numel() != H or not dw.is_contiguous()):
        raise ValueError("dw must be a contiguous float32 tensor of H elements")
    wcode = _dtype_code(weight) if weight is not None else _dtype_code(x)
    st = lib.rmsnorm_bwd_noalloc(_ptr(dy), dys, _ptr(x), xs, _ptr(weight), _ptr(rrms), _ptr(dx), dxs, _ptr(dw), M, H,
                                 _dtype_code(x), wcode, _stream(x))
    _check(lib, st)
    return dx, dw


def rmsnorm_bwd_residual(dy, residual_out, dres, weight, rrms, dh=None, dw=None, workspace=None,
                         want_dw: bool = True):
    """Gradients of the fused residual pre-norm (rmsnorm_fwd_residual).

    residual_out is the post-add stream h the forward wrote; dres is the
    gradient arriving on it (None when it feeds nothing).  Returns (dh, dw):
    dh = norm backward through h + dres is the gradient of both x and the
    residual input.  dh may be dy, residual_out or dres itself."""
    return _bwd(dy, residual_out, dres, weight, rrms, dh, dw, workspace, want_dw)


def _params(x, weight, bias, H):
    """w_dtype code for an optional weight and bias (one format, x's or float32)."""
    ref = weight if weight is not None else bias
    for name, t in (("weight", weight), ("bias", bias)):
        if t is not None and (t.numel() != H or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous tensor of H elements")
    if weight is not None and bias is not None and weight.dtype != bias.dtype:
        raise ValueError("weight and bias must share one dtype")
    return _dtype_code(ref) if ref is not None else _dtype_code(x)


def _stats(x, M, given, want):
    torch = _torch()
    if want and given is None:
        given = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    if given is not None and (given.dtype != torch.float32 or given.numel() != M or not given.is_contiguous()):
        raise ValueError("mean and rstd must be contiguous float32 tensors with one value per row")
    return given


def layernorm_fwd(x, weight=None, bias=None, eps: float = 1e-5, out=None, mean=None, rstd=None,
                  return_stats: bool = False):
    """LayerNorm over the last dim: (x - mean) / sqrt(var + eps) * weight + bias
    (population variance; weight and bias optional).  Returns y, or
    (y, mean, rstd) with return_stats."""
    torch = _torch()
    lib = load_library()
    M, H, xs = _rows(x, "x")
    if out is None:
        out = torch.empty_like(x, memory_format=torch.contiguous_format)
    if out.shape != x.shape or out.dtype != x.dtype:
        raise ValueError("out must match x in shape and dtype")
    _, _, ys = _rows(out, "out")
    mean, rstd = _stats(x, M, mean, return_stats), _stats(x, M, rstd, return_stats)
    wcode = _params(x, weight, bias, H)
    st = lib.layernorm_fwd(_ptr(x), xs, _ptr(weight), _ptr(bias), _ptr(out), ys, _ptr(mean), _ptr(rstd), M, H,
                           float(eps), _dtype_code(x), wcode, _stream(x))
    _check(lib, st)
    return (out, mean, rstd) if return_stats else out


def layernorm_fwd_residual(x, residual, weight=None, bias=None, eps: float = 1e-5, out=None, residual_out=None,
                           mean=None, rstd=None, return_stats: bool = False, write_residual: bool = True):
    """h = x + residual (float32; written to residual_out in x's dtype) and
    y = LayerNorm(h) of the unrounded sum.  Returns (y, residual_out), plus
    (mean, rstd) with return_stats.  residual_out may be `residual` itself."""
    torch = _torch()
    lib = load_library()
    M, H, xs = _rows(x, "x")
    if residual.shape != x.shape or residual.dtype != x.dtype:
        raise ValueError("residual must match x in shape and dtype")
    _, _, rs = _rows(residual, "residual")
    if out is None:
        out = torch.empty_like(x, memory_format=torch.contiguous_format)
    if out.shape != x.shape or out.dtype != x.dtype:
        raise ValueError("out must match x in shape and dtype")
    _, _, ys = _rows(out, "out")
    if write_residual and residual_out is None:
        residual_out = torch.empty_like(x, memory_format=torch.contiguous_format)
    ros = 0
    if residual_out is not None:
        if residual_out.shape != x.shape or residual_out.dtype != x.dtype:
            raise ValueError("residual_out must match x in shape and dtype")
        _, _, ros = _rows(residual_out, "residual_out")
    mean, rstd = _stats(x, M, mean, return_stats), _stats(x, M, rstd, return_stats)
    wcode = _params(x, weight, bias, H)
    st = lib.layernorm_fwd_residual(_ptr(x), xs, _ptr(residual), rs, _ptr(weight), _ptr(bias), _ptr(out), ys,
                                    _ptr(residual_out), ros, _ptr(mean), _ptr(rstd), M, H, float(eps),
                                    _dtype_code(x), wcode, _stream(x))
    _check(lib, st)
    res = (out, residual_out)
    return res + (mean, rstd) if return_stats else res


def _heads_view(t, name):
    """(batch, seq_len, heads, head_dim, row stride, head stride) of a
    [batch, seq_len, heads, head_dim] tensor whose batch and position axes
    collapse into rows of one stride (token b, s is row b * seq_len + s)."""
    if t.dim() != 4:
        raise ValueError(f"{name} must be [batch, seq_len, heads, head_dim]")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    B, S, NH, D = t.shape
    hs = t.stride(2) if NH > 1 else D
    span = (NH - 1) * hs + D  # elements of one token row
    if t.numel() == 0:
        return B, S, NH, D, max(span, 1), max(hs, 1)
    if t.stride(3) != 1 and D > 1:
        raise ValueError(f"{name} must be contiguous along head_dim")
    if S > 1:
        rs = t.stride(1)
        if B > 1 and t.stride(0) != S * rs:
            raise ValueError(f"{name}'s batch and position axes cannot be viewed as rows with one stride")
    else:
        rs = t.stride(0) if B > 1 else span
    return B, S, NH, D, rs, hs


def rope_apply(x, cos, sin, out=None, transpose: bool = False):
    """Rotate-half RoPE of x [batch, seq_len, heads, head_dim] by per-position
    cos/sin tables [seq_len, >= head_dim/2] (x's dtype or float32); token b, s
    reads table row s.  out may be x itself (in place).  transpose rotates by
    the negated angles (the inverse, and the gradient with respect to x)."""
    torch = _torch()
    lib = load_library()
    B, S, NH, D, xrs, xhs = _heads_view(x, "x")
    if out is None:
        out = torch.empty_like(x, memory_format=torch.contiguous_format)
    if out.shape != x.shape or out.dtype != x.dtype:
        raise ValueError("out must match x in shape and dtype")
    _, _, _, _, ors, ohs = _heads_view(out, "out")
    if cos.shape != sin.shape or cos.dtype != sin.dtype or cos.dim() != 2 or cos.shape[0] != S:
        raise ValueError("cos and sin must both be [seq_len, >= head_dim/2] tensors of one dtype")
    if cos.shape[1] < D // 2:
        raise ValueError("cos/sin rows must hold at least head_dim/2 entries")
    if cos.stride(1) != 1 or sin.stride(1) != 1 or (S > 1 and cos.stride(0) != sin.stride(0)):
        raise ValueError("cos and sin must be row-contiguous with one row stride")
    ts = cos.stride(0) if S > 1 else cos.shape[1]
    st = lib.rope_apply(_ptr(x), xrs, xhs, _ptr(cos), _ptr(sin), ts, _ptr(out), ors, ohs, B, S, NH, D,
                        1 if transpose else 0, _dtype_code(x), _dtype_code(cos), _stream(x))
    _check(lib, st)
    return out


def set_geometry(which: str, vpt: int = 0, wpr: int = 0, third: int = 0, grid: int = 0) -> None:
    """Development hook (include/rmsnorm_tuning.h): force the launch geometry
    of the forward ("fwd"), backward ("bwd") or RoPE ("rope") kernels; vpt=0 restores the
    library's own choice."""
    code = {"fwd": 0, "bwd": 1, "rope": 2}[which]
    load_library().rmsnorm_tuning_set_geometry(code, int(vpt), int(wpr), int(third), int(grid))


_TILE_OPS = {"fwd": 0, "fwd_residual": 1, "adaln": 2, "layernorm": 3, "bwd": 4, "bwd_residual": 5,
             "layernorm_residual": 6}
_DTYPE_NAMES = {"f32": 0, "f16": 1, "bf16": 2}


def tile(op: str, H: int, dtype: str, off_grid: bool, shared_offset: bool = False) -> dict:
    """Development hook (include/rmsnorm_tuning.h), host only: the register
    tile the library picks for `op` at row length H in `dtype` ("f32", "f16",
    "bf16"), for rows on the 16-byte grid (off_grid False) or rows whose
    starts are only element-aligned (True); shared_offset: off the grid, with
    every row stream of a backward at one offset within its 16-byte chunks
    ("frame": the backward's vectors then sit on memory's 16-byte grid)."""
    lib = load_library()
    out = (ctypes.c_int32 * 6)()
    layout = (2 if shared_offset else 1) if off_grid else 0
    _check(lib, lib.rmsnorm_tuning_tile(_TILE_OPS[op], int(H), _DTYPE_NAMES[dtype], layout, out))
    return {"vec": out[0], "vpt": out[1], "wpr": out[2], "rpw": out[3], "mis": bool(out[4]),
            "frame": out[4] == 2, "multi_pass": bool(out[5])}


def copy_reference(src, dst) -> None:
    """Development hook (include/rmsnorm_tuning.h): copy src into dst (same
    byte size, both contiguous device tensors) with the forward kernels'
    access pattern and no arithmetic -- the speed-of-light reference for a
    transfer of that size."""
    lib = load_library()
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes or not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("src and dst must be contiguous tensors of the same byte size")
    if not (src.is_cuda and dst.is_cuda):
        raise ValueError("src and dst must be device tensors")
    _check(lib, lib.rmsnorm_tuning_copy(_ptr(src), _ptr(dst), nbytes, _stream(src)))


def set_streaming(mode: int = -1) -> None:
    """Development hook (include/rmsnorm_tuning.h): -1 lets the library decide
    by size whether to stream inputs/outputs past the caches, 0 never, 1 always."""
    load_library().rmsnorm_tuning_set_streaming(int(mode))
