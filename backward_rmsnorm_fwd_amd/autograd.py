"""RMSNorm as a differentiable PyTorch operation over the C ABI.

The operation follows the page "Check an AI model calculation before
accelerating it", section "Connecting Autograd and actually training":

* the forward keeps x, the weight and the per-row inverse RMS for the
  backward, so eps is not needed again;
* the backward takes dy (made contiguous unless its rows are evenly
  strided), computes dx and the weight gradient
  with the library's two backward stages; the weight gradient comes out in
  the weight's dtype (the library rounds its float32 sum once);
* eps and the offset flag are not differentiated.

Both passes run the HIP kernels through ``rmsnorm_fwd`` / ``rmsnorm_bwd``.
There is no CPU path: CPU tensors or a missing library raise.

``CALLS`` counts passes through this wrapper (one count per forward and per
backward, whatever the number of kernel launches), so a training loop can
prove that the custom path, and not another implementation, took part.

The same wrapping is given to the library's other paths: LayerNorm
(``layernorm``, ``LayerNorm``), RMSNorm with the residual add fused before
it (``add_rmsnorm``, ``AddRMSNorm``: returns y and the new residual stream
h, both differentiable) and RMSNorm with its output cast to bf16/fp16
(``rmsnorm_cast``, ``RMSNormCast``).  Their passes are counted under their
own keys of ``CALLS``.
"""
from __future__ import annotations

import torch

from . import add_bwd as _add_bwd
from . import add_fwd as _add_fwd
from . import bwd as _bwd
from . import cast_bwd as _cast_bwd
from . import cast_fwd as _cast_fwd
from . import fwd as _fwd
from . import ln_bwd as _ln_bwd
from . import ln_fwd as _ln_fwd
from . import row_layout

__all__ = ["CALLS", "RMSNormFunction", "rmsnorm", "RMSNorm", "LayerNormFunction", "layernorm",
           "LayerNorm", "AddRMSNormFunction", "add_rmsnorm", "AddRMSNorm",
           "RMSNormCastFunction", "rmsnorm_cast", "RMSNormCast"]

CALLS = {"forward": 0, "backward": 0, "ln_forward": 0, "ln_backward": 0, "add_forward": 0,
         "add_backward": 0, "cast_forward": 0, "cast_backward": 0}


def _rows(t):
    """t itself when the library can read its rows, else a contiguous copy."""
    return t if row_layout(t) is not None else t.contiguous()


class RMSNormFunction(torch.autograd.Function):
    """y = x * rsqrt(mean(x^2) + eps) * g over the last dimension, where
    g = weight or g = 1 + weight (offset)."""

    @staticmethod
    def forward(ctx, x, weight, eps, offset):
        # The library reads rows at any row stride; other layouts are copied
        # once here.
        xc = x if row_layout(x) is not None else x.contiguous()
        y, rstd = _fwd(xc, weight, eps, offset)
        ctx.save_for_backward(xc, weight, rstd)
        ctx.offset = bool(offset)
        CALLS["forward"] += 1
        return y

    @staticmethod
    def backward(ctx, dy):
        xc, weight, rstd = ctx.saved_tensors
        dx, dgamma = _bwd(dy, xc, weight, rstd, ctx.offset, dgamma_dtype=weight.dtype)
        CALLS["backward"] += 1
        return dx, (dgamma if ctx.needs_input_grad[1] else None), None, None


def rmsnorm(x, weight, eps=1e-6, offset=False):
    """Differentiable RMSNorm of ``x`` over its last dimension."""
    return RMSNormFunction.apply(x, weight, eps, offset)


class RMSNorm(torch.nn.Module):
    """Module form.  With ``offset`` the learned parameter w starts at 0 and
    the applied weight is 1 + w; otherwise the weight starts at 1."""

    def __init__(self, dim, eps=1e-6, offset=False, device=None, dtype=None):
        super().__init__()
        init = torch.zeros if offset else torch.ones
        self.weight = torch.nn.Parameter(init(dim, device=device, dtype=dtype))
        self.eps = eps
        self.offset = offset

    def forward(self, x):
        return rmsnorm(x, self.weight, self.eps, self.offset)

    def extra_repr(self):
        return f"{self.weight.shape[0]}, eps={self.eps}, offset={self.offset}"


class LayerNormFunction(torch.autograd.Function):
    """y = (x - mean) * rsqrt(var + eps) * weight + bias over the last
    dimension (biased variance); bias may be None."""

    @staticmethod
    def forward(ctx, x, weight, bias, eps):
        xc = _rows(x)
        y, mean, rstd = _ln_fwd(xc, weight, bias, eps)
        ctx.save_for_backward(xc, weight, mean, rstd)
        ctx.has_bias = bias is not None
        CALLS["ln_forward"] += 1
        return y

    @staticmethod
    def backward(ctx, dy):
        xc, weight, mean, rstd = ctx.saved_tensors
        dx, dgamma, dbeta = _ln_bwd(dy, xc, weight, mean, rstd, dgamma_dtype=weight.dtype,
                                    bias=ctx.has_bias)
        CALLS["ln_backward"] += 1
        return (dx, dgamma if ctx.needs_input_grad[1] else None,
                dbeta if ctx.has_bias and ctx.needs_input_grad[2] else None, None)


def layernorm(x, weight, bias=None, eps=1e-5):
    """Differentiable LayerNorm of ``x`` over its last dimension."""
    return LayerNormFunction.apply(x, weight, bias, eps)


class LayerNorm(torch.nn.Module):
    """Module form: weight starts at 1, bias (when kept) at 0."""

    def __init__(self, dim, eps=1e-5, bias=True, device=None, dtype=None):
        super().__init__()
        self.weight = torch.nn.Parameter(torch.ones(dim, device=device, dtype=dtype))
        self.bias = (torch.nn.Parameter(torch.zeros(dim, device=device, dtype=dtype))
                     if bias else None)
        self.eps = eps

    def forward(self, x):
        return layernorm(x, self.weight, self.bias, self.eps)

    def extra_repr(self):
        return f"{self.weight.shape[0]}, eps={self.eps}, bias={self.bias is not None}"


class AddRMSNormFunction(torch.autograd.Function):
    """h = x + res (the dtype's add), y = RMSNorm(h).  Returns (y, h); the
    gradient reaching x and res is dRMSNorm/dh (dy) + dh."""

    @staticmethod
    def forward(ctx, x, res, weight, eps, offset):
        ctx.set_materialize_grads(False)
        y, h, rstd = _add_fwd(_rows(x), _rows(res), weight, eps, offset)
        ctx.save_for_backward(h, weight, rstd)
        ctx.offset = bool(offset)
        CALLS["add_forward"] += 1
        return y, h

    @staticmethod
    def backward(ctx, dy, dh):
        h, weight, rstd = ctx.saved_tensors
        if dy is None:
            dy = torch.zeros_like(h)
        dx, dgamma = _add_bwd(dy, dh, h, weight, rstd, ctx.offset, dgamma_dtype=weight.dtype)
        CALLS["add_backward"] += 1
        dres = None
        if ctx.needs_input_grad[1]:
            dres = dx.clone() if ctx.needs_input_grad[0] else dx
        return (dx if ctx.needs_input_grad[0] else None, dres,
                dgamma if ctx.needs_input_grad[2] else None, None, None)


def add_rmsnorm(x, res, weight, eps=1e-6, offset=False):
    """Differentiable ``(RMSNorm(x + res), x + res)`` over the last dimension."""
    return AddRMSNormFunction.apply(x, res, weight, eps, offset)


class AddRMSNorm(torch.nn.Module):
    """Module form of ``add_rmsnorm``: ``forward(x, res) -> (y, h)``."""

    def __init__(self, dim, eps=1e-6, offset=False, device=None, dtype=None):
        super().__init__()
        init = torch.zeros if offset else torch.ones
        self.weight = torch.nn.Parameter(init(dim, device=device, dtype=dtype))
        self.eps = eps
        self.offset = offset

    def forward(self, x, res):
        return add_rmsnorm(x, res, self.weight, self.eps, self.offset)


class RMSNormCastFunction(torch.autograd.Function):
    """y = T_out(RMSNorm(x)) for float32 x and weight; the gradient of y
    (in T_out) reaches x widened."""

    @staticmethod
    def forward(ctx, x, weight, out_dtype, eps, offset):
        xc = _rows(x)
        y, rstd = _cast_fwd(xc, weight, out_dtype, eps, offset)
        ctx.save_for_backward(xc, weight, rstd)
        ctx.offset = bool(offset)
        CALLS["cast_forward"] += 1
        return y

    @staticmethod
    def backward(ctx, dy):
        xc, weight, rstd = ctx.saved_tensors
        dx, dgamma = _cast_bwd(dy, xc, weight, rstd, ctx.offset)
        CALLS["cast_backward"] += 1
        return dx, (dgamma if ctx.needs_input_grad[1] else None), None, None, None


def rmsnorm_cast(x, weight, out_dtype=torch.bfloat16, eps=1e-6, offset=False):
    """Differentiable RMSNorm of float32 ``x`` with its output in ``out_dtype``."""
    return RMSNormCastFunction.apply(x, weight, out_dtype, eps, offset)


class RMSNormCast(torch.nn.Module):
    """Module form of ``rmsnorm_cast`` (float32 weight)."""

    def __init__(self, dim, out_dtype=torch.bfloat16, eps=1e-6, offset=False, device=None):
        super().__init__()
        init = torch.zeros if offset else torch.ones
        self.weight = torch.nn.Parameter(init(dim, device=device, dtype=torch.float32))
        self.out_dtype = out_dtype
        self.eps = eps
        self.offset = offset

    def forward(self, x):
        return rmsnorm_cast(x, self.weight, self.out_dtype, self.eps, self.offset)
