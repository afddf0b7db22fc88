"""Same-dtype eager reference on the CPU (test infrastructure only).

The "reference" of the torchtitan kernel-numerics-verifier page (section
"核心方法"): an eager implementation whose inputs and outputs have the kernel's
dtype and whose intermediates are float32.  Its distance to the float64 golden
(``reference_error``) calibrates how much error a correct implementation at
this precision makes; the gate lets the kernel have at most a fixed multiple of
it (see ``oracle.gate``).

The forward follows ``rmsnorm_reference`` and the backward the explicit
``manual_backward`` formula of the page "Check an AI model calculation before
accelerating it", section "PyTorch reference: the numerical oracle", with the
inputs promoted to float32 first (section "Why convert before reducing?").
Offset mode forms ``1 + w`` after promotion to float32, as the torchtitan
page's ``_offset_rms_norm_reference`` does.  rstd and dgamma are float32.

``reference_backward_autograd`` is the torchtitan page's variant (autograd of
the eager float32 formula); it is logged beside the explicit formula, while the
explicit formula is the one that gates.
"""
from __future__ import annotations

import torch

DEFAULT_EPS = 1e-6


def _rows2d(t):
    return t.reshape(1, -1) if t.dim() == 1 else t.reshape(-1, t.shape[-1])


def _weight32(weight, offset):
    g = weight.detach().to("cpu").float().reshape(-1)
    return 1.0 + g if offset else g


def reference_forward(x, weight, eps=DEFAULT_EPS, offset=False):
    """Returns ``(y, rstd)``: y in x's dtype [M, N], rstd float32 [M]."""
    x2 = _rows2d(x.detach().to("cpu"))
    xf = x2.float()
    g = _weight32(weight, offset)
    r = torch.rsqrt(xf.square().mean(-1, keepdim=True) + eps)
    y = (xf * r * g).to(x.dtype)
    return y, r.squeeze(-1)


def reference_backward(dy, x, weight, eps=DEFAULT_EPS, offset=False):
    """Explicit float32 backward.  Returns ``(dx, dgamma)``.

    dx has x's dtype [M, N]; dgamma is float32 [N] (a sum over rows).
    """
    x2 = _rows2d(x.detach().to("cpu"))
    dy2 = _rows2d(dy.detach().to("cpu"))
    xf = x2.float()
    dyf = dy2.float()
    g = _weight32(weight, offset)
    r = torch.rsqrt(xf.square().mean(-1, keepdim=True) + eps)
    u = dyf * g
    dx = r * u - xf * r.pow(3) * (u * xf).mean(-1, keepdim=True)
    dgamma = (dyf * xf * r).sum(0)
    return dx.to(x.dtype), dgamma


def reference_dgamma(dy, x, eps=DEFAULT_EPS, cols=None):
    """dgamma of ``reference_backward`` restricted to some columns.

    Same float32 arithmetic: r from whole rows, then (dy*x*r) summed over
    rows for the selected columns only."""
    x2 = _rows2d(x.detach().to("cpu"))
    dy2 = _rows2d(dy.detach().to("cpu"))
    xf = x2.float()
    r = torch.rsqrt(xf.square().mean(-1, keepdim=True) + eps)
    if cols is not None:
        idx = torch.as_tensor(cols, dtype=torch.long)
        xf = xf[:, idx]
        dyf = dy2[:, idx].float()
    else:
        dyf = dy2.float()
    return (dyf * xf * r).sum(0)


def reference_backward_autograd(dy, x, weight, eps=DEFAULT_EPS, offset=False):
    """Autograd of the float32 eager forward (informational only)."""
    x2 = _rows2d(x.detach().to("cpu"))
    dy2 = _rows2d(dy.detach().to("cpu"))
    xf = x2.float().requires_grad_(True)
    w = weight.detach().to("cpu").float().reshape(-1).requires_grad_(True)
    g = 1.0 + w if offset else w
    r = torch.rsqrt(xf.square().mean(-1, keepdim=True) + eps)
    y = xf * r * g
    dx, dw = torch.autograd.grad(y, (xf, w), dy2.float())
    return dx.to(x.dtype), dw
