"""Same-dtype eager reference on the CPU (test infrastructure only).

The "reference" of the torchtitan kernel-numerics-verifier page (section
"核心方法"): an eager implementation whose inputs and outputs have the kernel's
dtype and whose intermediates are float32.  Its distance to the float64 golden
(``reference_error``) calibrates how much error a correct implementation at
this precision makes; the gate lets the kernel have at most a fixed multiple of
it (see ``oracle.gate``).

The arithmetic is the definition of RMSNorm and of its exact gradient, as the
page "Check an AI model calculation before accelerating it" states them
(sections "Problem and reference formula", "Input backward pass: keep the
right N" and "A sum is not an average"), evaluated in float32 after the
inputs are promoted (section "Why convert before reducing?"):

* ``ss = sum_j x_j^2``, ``r = 1/sqrt(ss/N + eps)``, ``xhat = x*r``,
  ``y = xhat*g``;
* ``u = dy*g``, ``c = sum_j u_j*x_j / N``, ``dx = r*(u - x*r^2*c)``;
* ``dgamma_j = sum_i dy_ij*x_ij*r_i``, products taken left to right as the
  formula is written.

Offset mode forms ``g = 1 + w`` after promotion to float32, as the torchtitan
page's offset reference does.  rstd and dgamma are float32.

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


def _row_rstd32(xf, eps):
    """Per-row r = 1/sqrt(sum(x^2)/N + eps) in float32, kept as a column."""
    n = xf.shape[-1]
    ss = (xf * xf).sum(-1, keepdim=True)
    return torch.rsqrt(ss / n + eps)


def _column_sums32(t):
    """float32 sums over the rows of t, one per column.  Each column is summed
    as its own contiguous vector, so its result does not depend on which other
    columns are summed beside it."""
    return t.t().contiguous().sum(-1)


def reference_forward(x, weight, eps=DEFAULT_EPS, offset=False):
    """Returns ``(y, rstd)``: y in x's dtype [M, N], rstd float32 [M]."""
    xf = _rows2d(x.detach().to("cpu")).float()
    g = _weight32(weight, offset)
    r = _row_rstd32(xf, eps)
    y = (xf * r) * g
    return y.to(x.dtype), r.squeeze(-1)


def reference_backward(dy, x, weight, eps=DEFAULT_EPS, offset=False):
    """Explicit float32 backward.  Returns ``(dx, dgamma)``.

    dx has x's dtype [M, N]; dgamma is float32 [N] (a sum over rows).
    """
    xf = _rows2d(x.detach().to("cpu")).float()
    dyf = _rows2d(dy.detach().to("cpu")).float()
    g = _weight32(weight, offset)
    n = xf.shape[-1]
    r = _row_rstd32(xf, eps)
    u = dyf * g
    c = (u * xf).sum(-1, keepdim=True) / n
    dx = r * (u - xf * (r * r) * c)
    dgamma = _column_sums32(dyf * xf * r)
    return dx.to(x.dtype), dgamma


def reference_dgamma(dy, x, eps=DEFAULT_EPS, cols=None):
    """dgamma of ``reference_backward`` restricted to some columns.

    Same float32 arithmetic: r from whole rows, then dy*x*r (left to right)
    summed over rows for the selected columns only."""
    xf = _rows2d(x.detach().to("cpu")).float()
    dy2 = _rows2d(dy.detach().to("cpu"))
    r = _row_rstd32(xf, eps)
    if cols is not None:
        idx = torch.as_tensor(cols, dtype=torch.long)
        xf = xf[:, idx]
        dy2 = dy2[:, idx]
    return _column_sums32(dy2.float() * xf * r)


def reference_backward_autograd(dy, x, weight, eps=DEFAULT_EPS, offset=False):
    """Autograd of the float32 eager forward (informational only)."""
    x2 = _rows2d(x.detach().to("cpu"))
    dy2 = _rows2d(dy.detach().to("cpu"))
    xf = x2.float().requires_grad_(True)
    w = weight.detach().to("cpu").float().reshape(-1).requires_grad_(True)
    g = 1.0 + w if offset else w
    y = (xf * _row_rstd32(xf, eps)) * g
    dx, dw = torch.autograd.grad(y, (xf, w), dy2.float())
    return dx.to(x.dtype), dw
