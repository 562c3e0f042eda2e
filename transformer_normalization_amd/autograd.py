"""Training integration: torch.autograd Functions and nn.Modules over the
library's C ABI.

    y = rms_norm(x, weight, eps)                        # differentiable
    y, h = fused_add_rms_norm(x, residual, weight, eps)  # h = x + residual
    norm = RMSNorm(4096, eps=1e-5, device="cuda", dtype=torch.bfloat16)
    y = norm(x);  y, h = norm(x, residual)
    q = rope_3d(q, cos, sin)                            # differentiable in q

RoPE's backward is the transposed rotation (the same kernel with the sine
negated); the tables are constants (no gradient).

The forward saves the per-row float32 rrms the forward kernel writes, and the
backward reads it instead of recomputing it (page "Skill: Write a Triton
RMSNorm Kernel", "Required reasoning process" step 10 and "Correctness
requirements").  The fused residual variant saves the post-add stream h it
wrote back and, in the backward, adds the gradient arriving on h to the
norm's input gradient inside the backward kernel, so the residual stream's
gradient costs no extra pass over memory.  The weight gradient is the
library's float32 dw, cast to the weight's dtype.

Every computation runs in the HIP kernels; these classes only marshal
tensors.  The library's outputs are new tensors (never views of the inputs),
and gradients have the inputs' shapes and dtypes.
"""

from __future__ import annotations

import torch

from . import rmsnorm_bwd, rmsnorm_bwd_residual, rmsnorm_fwd, rmsnorm_fwd_residual, rope_apply

__all__ = ["RMSNormFunction", "FusedAddRMSNormFunction", "RoPEFunction", "rms_norm", "fused_add_rms_norm", "rope_3d",
           "RMSNorm"]


def _grad_like(g, ref):
    """Incoming gradient as a tensor the library can read: ref's dtype, unit
    stride along the last dim (expanded or transposed gradients are copied)."""
    if g.dtype != ref.dtype:
        g = g.to(ref.dtype)
    if g.shape != ref.shape:
        g = g.expand(ref.shape)
    return g.contiguous()


class RMSNormFunction(torch.autograd.Function):
    """y = x * rsqrt(mean(x^2, -1) + eps) * weight (weight may be None)."""

    @staticmethod
    def forward(ctx, x, weight, eps):
        y, rrms = rmsnorm_fwd(x, weight, eps, return_rrms=True)
        ctx.save_for_backward(x, weight, rrms)
        ctx.has_weight = weight is not None
        return y

    @staticmethod
    def backward(ctx, dy):
        x, weight, rrms = ctx.saved_tensors
        want_dw = ctx.has_weight and ctx.needs_input_grad[1]
        dx, dw = rmsnorm_bwd(_grad_like(dy, x), x, weight if ctx.has_weight else None, rrms, want_dw=want_dw)
        if dw is not None:
            dw = dw.to(weight.dtype).view(weight.shape)
        return (dx if ctx.needs_input_grad[0] else None), dw, None


class FusedAddRMSNormFunction(torch.autograd.Function):
    """(y, h) with h = x + residual (float32 sum, stored in x's dtype) and
    y = RMSNorm(h) of the unrounded sum; x and residual both receive
    dL/dh = norm backward + the gradient arriving on h."""

    @staticmethod
    def forward(ctx, x, residual, weight, eps):
        y, h, rrms = rmsnorm_fwd_residual(x, residual, weight, eps, return_rrms=True)
        ctx.save_for_backward(h, weight, rrms)
        ctx.has_weight = weight is not None
        # a gradient that is never produced for h stays None (no zero tensor)
        ctx.set_materialize_grads(False)
        return y, h

    @staticmethod
    def backward(ctx, dy, dh_in):
        h, weight, rrms = ctx.saved_tensors
        w = weight if ctx.has_weight else None
        want_dw = ctx.has_weight and ctx.needs_input_grad[2]
        if dy is None:
            # only h reaches the loss: the norm contributes nothing
            dres = _grad_like(dh_in, h)
            dw = torch.zeros_like(weight) if want_dw else None
            return dres, dres, dw, None
        dres = None if dh_in is None else _grad_like(dh_in, h)
        dh, dw = rmsnorm_bwd_residual(_grad_like(dy, h), h, dres, w, rrms, want_dw=want_dw)
        if dw is not None:
            dw = dw.to(weight.dtype).view(weight.shape)
        gx = dh if ctx.needs_input_grad[0] else None
        gr = dh if ctx.needs_input_grad[1] else None
        return gx, gr, dw, None


class RoPEFunction(torch.autograd.Function):
    """Rotate-half RoPE of q or k [batch, seq_len, heads, head_dim] by
    [seq_len, head_dim] cos/sin tables (constants)."""

    @staticmethod
    def forward(ctx, x, cos, sin):
        ctx.save_for_backward(cos, sin)
        return rope_apply(x, cos, sin)

    @staticmethod
    def backward(ctx, dy):
        cos, sin = ctx.saved_tensors
        if ctx.needs_input_grad[1] or ctx.needs_input_grad[2]:
            raise NotImplementedError("rope_3d has no gradient with respect to the cos/sin tables")
        return rope_apply(_grad_like(dy, dy), cos, sin, transpose=True), None, None


def rms_norm(x, weight=None, eps: float = 1e-6):
    """Differentiable RMSNorm over the last dimension of x."""
    return RMSNormFunction.apply(x, weight, eps)


def fused_add_rms_norm(x, residual, weight=None, eps: float = 1e-6):
    """Differentiable fused residual pre-norm: returns (RMSNorm(x + residual), x + residual)."""
    return FusedAddRMSNormFunction.apply(x, residual, weight, eps)


def rope_3d(x, cos, sin):
    """Differentiable rotate-half RoPE (gradient with respect to x only)."""
    return RoPEFunction.apply(x, cos, sin)


class RMSNorm(torch.nn.Module):
    """RMSNorm layer over the trailing `hidden_size` dimension.

    forward(x) -> y;  forward(x, residual) -> (y, x + residual), the fused
    pre-norm of a transformer block whose second output is the next residual
    stream.  elementwise_affine=False gives the weightless norm."""

    def __init__(self, hidden_size: int, eps: float = 1e-6, elementwise_affine: bool = True, device=None,
                 dtype=None):
        super().__init__()
        self.hidden_size = int(hidden_size)
        self.eps = float(eps)
        if elementwise_affine:
            self.weight = torch.nn.Parameter(torch.ones(self.hidden_size, device=device, dtype=dtype))
        else:
            self.register_parameter("weight", None)

    def forward(self, x, residual=None):
        if x.shape[-1] != self.hidden_size:
            raise ValueError(f"last dimension {x.shape[-1]} != hidden_size {self.hidden_size}")
        if residual is None:
            return rms_norm(x, self.weight, self.eps)
        return fused_add_rms_norm(x, residual, self.weight, self.eps)

    def extra_repr(self):
        return f"{self.hidden_size}, eps={self.eps}, elementwise_affine={self.weight is not None}"
