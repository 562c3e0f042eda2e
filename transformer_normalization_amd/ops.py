"""The library's operations registered as torch custom operators
(torch.library.custom_op, namespace "tn"), with fake (shape) implementations
and autograd formulas, so that torch.compile and other graph capture treat
each call as one opaque node instead of breaking the graph at the ctypes
call.

    torch.ops.tn.rms_norm(x, weight, eps)                   -> y
    torch.ops.tn.fused_add_rms_norm(x, residual, weight, eps) -> (y, h)
    torch.ops.tn.rope(x, cos, sin, transpose)              -> out
    torch.ops.tn.adaln_rms_norm(x, weight, scale, shift, eps) -> y      (no gradient)
    torch.ops.tn.layer_norm_residual(x, residual, weight, bias, eps) -> (y, h)  (no gradient)

The backward of rms_norm and fused_add_rms_norm reads the float32 rrms the
forward saved, as the autograd Functions of transformer_normalization_amd.autograd
do; every computation runs in the library's HIP kernels.
"""

from __future__ import annotations

from typing import Optional

import torch
from torch import Tensor

from . import (layernorm_fwd_residual, rmsnorm_adaln_fwd, rmsnorm_bwd, rmsnorm_bwd_residual, rmsnorm_fwd,
               rmsnorm_fwd_residual, rope_apply)

__all__ = ["rms_norm", "fused_add_rms_norm", "rope", "adaln_rms_norm", "layer_norm_residual"]


def _rows_of(x: Tensor):
    return x.shape[:-1]


def _grad(g: Tensor, ref: Tensor) -> Tensor:
    if g.dtype != ref.dtype:
        g = g.to(ref.dtype)
    return g.expand(ref.shape).contiguous() if g.shape != ref.shape else g.contiguous()


# ---- RMSNorm ------------------------------------------------------------------

@torch.library.custom_op("tn::rms_norm_fwd", mutates_args=())
def _rms_norm_fwd(x: Tensor, weight: Optional[Tensor], eps: float) -> tuple[Tensor, Tensor]:
    y, rrms = rmsnorm_fwd(x.contiguous(), weight, eps, return_rrms=True)
    return y, rrms


@_rms_norm_fwd.register_fake
def _(x, weight, eps):
    return torch.empty_like(x, memory_format=torch.contiguous_format), x.new_empty(_rows_of(x), dtype=torch.float32)


@torch.library.custom_op("tn::rms_norm_bwd", mutates_args=())
def _rms_norm_bwd(dy: Tensor, x: Tensor, weight: Optional[Tensor], rrms: Tensor, dres: Optional[Tensor],
                  want_dw: bool) -> tuple[Tensor, Tensor]:
    """(dx, dw); dw is float32, empty when not wanted.  With dres, x is the
    stored post-add stream and dx includes dres (fused residual backward)."""
    if dres is None:
        dx, dw = rmsnorm_bwd(dy, x, weight, rrms, want_dw=want_dw)
    else:
        dx, dw = rmsnorm_bwd_residual(dy, x, dres, weight, rrms, want_dw=want_dw)
    return dx, (dw if dw is not None else x.new_empty((0,), dtype=torch.float32))


@_rms_norm_bwd.register_fake
def _(dy, x, weight, rrms, dres, want_dw):
    n = x.shape[-1] if (want_dw and weight is not None) else 0
    return torch.empty_like(x, memory_format=torch.contiguous_format), x.new_empty((n,), dtype=torch.float32)


def rms_norm(x: Tensor, weight: Optional[Tensor] = None, eps: float = 1e-6) -> Tensor:
    """Differentiable RMSNorm as a custom operator."""
    return _rms_norm_fwd(x, weight, eps)[0]


def _rms_norm_setup(ctx, inputs, output):
    x, weight, eps = inputs
    ctx.save_for_backward(x.contiguous(), weight, output[1])
    ctx.has_weight = weight is not None


def _rms_norm_backward(ctx, dy, drrms):
    x, weight, rrms = ctx.saved_tensors
    want_dw = ctx.has_weight and ctx.needs_input_grad[1]
    dx, dw = _rms_norm_bwd(_grad(dy, x), x, weight if ctx.has_weight else None, rrms, None, want_dw)
    return dx, (dw.to(weight.dtype) if want_dw else None), None


_rms_norm_fwd.register_autograd(_rms_norm_backward, setup_context=_rms_norm_setup)


# ---- fused residual pre-norm ---------------------------------------------------

@torch.library.custom_op("tn::fused_add_rms_norm", mutates_args=())
def _fused_fwd(x: Tensor, residual: Tensor, weight: Optional[Tensor], eps: float) -> tuple[Tensor, Tensor, Tensor]:
    y, h, rrms = rmsnorm_fwd_residual(x.contiguous(), residual.contiguous(), weight, eps, return_rrms=True)
    return y, h, rrms


@_fused_fwd.register_fake
def _(x, residual, weight, eps):
    e = torch.empty_like(x, memory_format=torch.contiguous_format)
    return e, torch.empty_like(e), x.new_empty(_rows_of(x), dtype=torch.float32)


def fused_add_rms_norm(x: Tensor, residual: Tensor, weight: Optional[Tensor] = None, eps: float = 1e-6):
    """(RMSNorm(x + residual), x + residual) as a custom operator."""
    y, h, _ = _fused_fwd(x, residual, weight, eps)
    return y, h


def _fused_setup(ctx, inputs, output):
    x, residual, weight, eps = inputs
    ctx.save_for_backward(output[1], weight, output[2])
    ctx.has_weight = weight is not None


def _fused_backward(ctx, dy, dh_in, drrms):
    h, weight, rrms = ctx.saved_tensors
    want_dw = ctx.has_weight and ctx.needs_input_grad[2]
    dres = None if dh_in is None else _grad(dh_in, h)
    dh, dw = _rms_norm_bwd(_grad(dy, h), h, weight if ctx.has_weight else None, rrms, dres, want_dw)
    return dh, dh, (dw.to(weight.dtype) if want_dw else None), None


_fused_fwd.register_autograd(_fused_backward, setup_context=_fused_setup)


# ---- RoPE ---------------------------------------------------------------------

@torch.library.custom_op("tn::rope", mutates_args=())
def _rope(x: Tensor, cos: Tensor, sin: Tensor, transpose: bool) -> Tensor:
    return rope_apply(x, cos, sin, transpose=transpose)


@_rope.register_fake
def _(x, cos, sin, transpose):
    return torch.empty_like(x, memory_format=torch.contiguous_format)


def rope(x: Tensor, cos: Tensor, sin: Tensor, transpose: bool = False) -> Tensor:
    """Rotate-half RoPE of x [batch, seq_len, heads, head_dim] as a custom operator."""
    return _rope(x, cos, sin, transpose)


def _rope_setup(ctx, inputs, output):
    x, cos, sin, transpose = inputs
    ctx.save_for_backward(cos, sin)
    ctx.transpose = transpose


def _rope_backward(ctx, dy):
    cos, sin = ctx.saved_tensors
    if ctx.needs_input_grad[1] or ctx.needs_input_grad[2]:
        raise NotImplementedError("tn::rope has no gradient with respect to the cos/sin tables")
    return _rope(_grad(dy, dy), cos, sin, not ctx.transpose), None, None, None


_rope.register_autograd(_rope_backward, setup_context=_rope_setup)


# ---- forward-only operators ------------------------------------------------------

@torch.library.custom_op("tn::adaln_rms_norm", mutates_args=())
def _adaln(x: Tensor, weight: Optional[Tensor], scale: Tensor, shift: Tensor, eps: float) -> Tensor:
    return rmsnorm_adaln_fwd(x.contiguous(), weight, scale, shift, eps)


@_adaln.register_fake
def _(x, weight, scale, shift, eps):
    return torch.empty_like(x, memory_format=torch.contiguous_format)


def adaln_rms_norm(x: Tensor, weight: Optional[Tensor], scale: Tensor, shift: Tensor, eps: float = 1e-6) -> Tensor:
    """AdaLN-RMSNorm, norm(x) * weight * (1 + scale) + shift (forward only)."""
    return _adaln(x, weight, scale, shift, eps)


@torch.library.custom_op("tn::layer_norm_residual", mutates_args=())
def _ln_residual(x: Tensor, residual: Tensor, weight: Optional[Tensor], bias: Optional[Tensor],
                 eps: float) -> tuple[Tensor, Tensor]:
    y, h = layernorm_fwd_residual(x.contiguous(), residual.contiguous(), weight, bias, eps)
    return y, h


@_ln_residual.register_fake
def _(x, residual, weight, bias, eps):
    e = torch.empty_like(x, memory_format=torch.contiguous_format)
    return e, torch.empty_like(e)


def layer_norm_residual(x: Tensor, residual: Tensor, weight: Optional[Tensor] = None, bias: Optional[Tensor] = None,
                        eps: float = 1e-5):
    """(LayerNorm(x + residual), x + residual) (forward only)."""
    return _ln_residual(x, residual, weight, bias, eps)
