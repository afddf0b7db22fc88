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
"""
from __future__ import annotations

import torch

from . import bwd as _bwd
from . import fwd as _fwd
from . import row_layout

__all__ = ["CALLS", "RMSNormFunction", "rmsnorm", "RMSNorm"]

CALLS = {"forward": 0, "backward": 0}


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
