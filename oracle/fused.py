"""Neighbours fused with RMSNorm -- TEST INFRASTRUCTURE ONLY.

The neighbour fused before the norm (the page "PyTorch torch.compile ...
LayerNorm and RMSNorm" argues, in its introduction, that a normalisation
kernel gains from fusing the operations around it; a transformer block adds
the sublayer output to the residual stream right before the norm).  The
fused operation is the composition a model runs unfused:

    h = T(x + residual)      PyTorch's add in the input dtype T: the float32
                             sum of the widened operands, rounded to nearest
                             even once (the new residual stream, kept)
    y = RMSNorm(h)           as in oracle.golden / oracle.reference

and its backward, with dh the gradient arriving on h from the residual
stream (None means 0):

    dx = dresidual = dRMSNorm/dh (dy) + dh      (one tensor serves both)
    dgamma         = the RMSNorm weight gradient at h

h is formed with PyTorch's own CPU add so it is exactly the tensor an
unfused model would normalise; everything after it reuses the pinned RMSNorm
golden (float64) and reference (float32) functions.

The neighbour fused after the norm is a cast of its output to a narrower
dtype (float32 in, bfloat16 or float16 out: a float32 residual stream feeding
a lower-precision consumer):

    y  = T_out(RMSNorm(x))   the norm in float32 as in oracle.reference,
                             then one round-to-nearest-even cast to T_out
                             (torch's ``.to``); the golden stays float64
    dx = dRMSNorm/dx (dy)    dy arrives in T_out; a dtype conversion passes
                             its gradient through unchanged (PyTorch's
                             convention), so dy is widened, exactly, and the
                             RMSNorm backward runs on it; dgamma likewise
"""
from __future__ import annotations

import numpy as np
import torch

from . import golden, reference


def residual_sum(x, residual):
    """h = x + residual in x's dtype, as PyTorch computes it on the CPU."""
    x = x.detach().to("cpu")
    residual = residual.detach().to("cpu")
    if x.dtype != residual.dtype or x.shape != residual.shape:
        raise ValueError("x and residual must share dtype and shape")
    return x + residual


def golden_add_forward(x, residual, weight, eps=golden.DEFAULT_EPS, offset=False, rows=None):
    """Returns ``(h, y, r)``: h in x's dtype (all rows), y and r float64."""
    h = residual_sum(x, residual)
    y, r = golden.golden_forward(h, weight, eps, offset, rows=rows)
    return h, y, r


def golden_add_dx(dy, dh, h, weight, eps=golden.DEFAULT_EPS, offset=False, rows=None):
    """float64 gradient of x (and of the residual) for all rows or ``rows``."""
    dx = golden.golden_dx(dy, h, weight, eps, offset, rows=rows)
    if dh is not None:
        d = golden._f64(golden._rows2d(dh))
        dx = dx + (d if rows is None else d[np.asarray(rows)])
    return dx


def golden_add_backward(dy, dh, h, weight, eps=golden.DEFAULT_EPS, offset=False):
    """Returns ``(dx, dgamma)`` in float64."""
    return (golden_add_dx(dy, dh, h, weight, eps, offset),
            golden.golden_dgamma(dy, h, eps))


def reference_add_forward(x, residual, weight, eps=reference.DEFAULT_EPS, offset=False):
    """Returns ``(h, y, rstd)``: h and y in x's dtype, rstd float32."""
    h = residual_sum(x, residual)
    y, r = reference.reference_forward(h, weight, eps, offset)
    return h, y, r


def reference_add_backward(dy, dh, h, weight, eps=reference.DEFAULT_EPS, offset=False):
    """float32 backward: the explicit RMSNorm formula at h, plus dh in
    float32, rounded once to the dtype.  Returns ``(dx, dgamma)``."""
    hf = reference._rows2d(h.detach().to("cpu")).float()
    dyf = reference._rows2d(dy.detach().to("cpu")).float()
    g = reference._weight32(weight, offset)
    r = torch.rsqrt(hf.square().mean(-1, keepdim=True) + eps)
    u = dyf * g
    dx = r * u - hf * r.pow(3) * (u * hf).mean(-1, keepdim=True)
    if dh is not None:
        dx = dx + reference._rows2d(dh.detach().to("cpu")).float()
    return dx.to(h.dtype), (dyf * hf * r).sum(0)


# ---- the output cast fused after the norm -----------------------------------

def golden_cast_forward(x, weight, eps=golden.DEFAULT_EPS, offset=False, rows=None):
    """float64 ``(y, r)``: the RMSNorm golden; a cast has no golden of its
    own (the gate compares the cast output with this exact value)."""
    return golden.golden_forward(x, weight, eps, offset, rows=rows)


def golden_cast_dx(dy, x, weight, eps=golden.DEFAULT_EPS, offset=False, rows=None):
    """float64 gradient of x: dy (in the narrow dtype) widened exactly."""
    return golden.golden_dx(dy, x, weight, eps, offset, rows=rows)


def golden_cast_backward(dy, x, weight, eps=golden.DEFAULT_EPS, offset=False):
    """Returns ``(dx, dgamma)`` in float64."""
    return golden.golden_backward(dy, x, weight, eps, offset)


def reference_cast_forward(x, weight, out_dtype, eps=reference.DEFAULT_EPS, offset=False):
    """Returns ``(y, rstd)``: the float32 reference norm, y rounded once to
    ``out_dtype``; rstd float32."""
    x2 = reference._rows2d(x.detach().to("cpu"))
    xf = x2.float()
    g = reference._weight32(weight, offset)
    r = torch.rsqrt(xf.square().mean(-1, keepdim=True) + eps)
    return (xf * r * g).to(out_dtype), r.squeeze(-1)


def reference_cast_backward(dy, x, weight, eps=reference.DEFAULT_EPS, offset=False):
    """float32 backward with dy widened from its narrow dtype.  Returns
    ``(dx, dgamma)``: dx in x's dtype, dgamma float32."""
    return reference.reference_backward(dy.detach().to("cpu").float(), x, weight, eps, offset)
