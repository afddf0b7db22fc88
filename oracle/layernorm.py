"""LayerNorm golden (float64) and same-dtype reference -- TEST INFRASTRUCTURE ONLY.

The sibling operation of RMSNorm on the page "PyTorch torch.compile ...
LayerNorm and RMSNorm" (itsolotime), section 1.1 (layer normalisation: each
row is normalised by its own mean and variance, then scaled by a learned
weight gamma and shifted by a learned bias beta) and section 2 (the backward
produces the input gradient, the weight gradient and, for LayerNorm only, the
bias gradient).  Section 1.4 has the forward keep the per-row statistics for
the backward; here they are the mean and the inverse standard deviation.

Definition, per row i of an M x N matrix (readings: the variance is the
biased one, divided by N like the mean; eps sits inside the square root as in
RMSNorm):

    mu_i    = (1/N) sum_j x_ij
    var_i   = (1/N) sum_j (x_ij - mu_i)^2
    r_i     = 1 / sqrt(var_i + eps)
    xhat_ij = (x_ij - mu_i) * r_i
    y_ij    = xhat_ij * gamma_j + beta_j

Backward (chain rule through mu_i and var_i; written out below and pinned by
central differences and by PyTorch's own layer_norm under autograd in
float64): with u_ij = dy_ij * gamma_j,

    dx_ij     = r_i * (u_ij - mean_j(u_ij) - xhat_ij * mean_j(u_ij * xhat_ij))
    dgamma_j  = sum_i dy_ij * xhat_ij
    dbeta_j   = sum_i dy_ij

``golden_*`` evaluate this in float64 with NumPy on the inputs promoted
losslessly; ``reference_*`` evaluate the same formulas with PyTorch on the CPU
in float32 after promotion (two passes over the row for the variance), with y
and dx rounded to the input dtype.  Neither imports anything from the HIP
library.
"""
from __future__ import annotations

import numpy as np
import torch

DEFAULT_EPS = 1e-6
CHUNK_ROWS = 4096


def _rows2d(a):
    if not hasattr(a, "ndim"):  # nested lists
        a = np.asarray(a, dtype=np.float64)
    return a.reshape(1, -1) if a.ndim == 1 else a.reshape(-1, a.shape[-1])


def _f64(a):
    if hasattr(a, "detach"):
        return a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def _check_eps(eps):
    if not (np.isfinite(eps) and eps > 0):
        raise ValueError("eps must be finite and positive")


def _stats(xc, eps):
    """(mu, r) of each row of a float64 chunk: mean, then the mean of the
    squared deviations from it."""
    n = xc.shape[1]
    mu = np.sum(xc, axis=1) / n
    d = xc - mu[:, None]
    var = np.sum(d * d, axis=1) / n
    return mu, 1.0 / np.sqrt(var + eps)


def _vec(v, n, name):
    a = np.zeros(n) if v is None else _f64(v).reshape(-1)
    if a.shape[0] != n:
        raise ValueError(f"{name} length must equal the row length N")
    return a


def golden_ln_forward(x, gamma, beta=None, eps=DEFAULT_EPS, rows=None,
                      chunk_rows=CHUNK_ROWS):
    """Returns ``(y, mean, rstd)`` in float64 for all rows or ``rows``.
    ``beta=None`` means no bias."""
    _check_eps(eps)
    x2 = _rows2d(x)
    n = x2.shape[1]
    g = _vec(gamma, n, "gamma")
    b = _vec(beta, n, "beta")
    idx = np.arange(x2.shape[0]) if rows is None else np.asarray(rows)
    y = np.empty((len(idx), n))
    mean = np.empty(len(idx))
    rstd = np.empty(len(idx))
    for lo in range(0, len(idx), chunk_rows):
        sel = idx[lo:lo + chunk_rows]
        xc = _f64(x2[sel])
        mu, r = _stats(xc, eps)
        y[lo:lo + len(sel)] = (xc - mu[:, None]) * r[:, None] * g[None, :] + b[None, :]
        mean[lo:lo + len(sel)] = mu
        rstd[lo:lo + len(sel)] = r
    return y, mean, rstd


def golden_ln_dx(dy, x, gamma, eps=DEFAULT_EPS, rows=None, chunk_rows=CHUNK_ROWS):
    """Input gradient (float64 [R, N]) for all rows or ``rows``."""
    _check_eps(eps)
    x2, dy2 = _rows2d(x), _rows2d(dy)
    if dy2.shape != x2.shape:
        raise ValueError("dy must have the shape of x")
    n = x2.shape[1]
    g = _vec(gamma, n, "gamma")
    idx = np.arange(x2.shape[0]) if rows is None else np.asarray(rows)
    dx = np.empty((len(idx), n))
    for lo in range(0, len(idx), chunk_rows):
        sel = idx[lo:lo + chunk_rows]
        xc, dyc = _f64(x2[sel]), _f64(dy2[sel])
        mu, r = _stats(xc, eps)
        xhat = (xc - mu[:, None]) * r[:, None]
        u = dyc * g[None, :]
        mu_u = np.sum(u, axis=1, keepdims=True) / n
        mu_ux = np.sum(u * xhat, axis=1, keepdims=True) / n
        dx[lo:lo + len(sel)] = r[:, None] * (u - mu_u - xhat * mu_ux)
    return dx


def golden_ln_param_grads(dy, x, eps=DEFAULT_EPS, cols=None, chunk_rows=CHUNK_ROWS):
    """``(dgamma, dbeta)`` in float64: column sums over ALL rows of dy*xhat
    and of dy, for all columns or ``cols`` (the statistics still come from
    whole rows)."""
    _check_eps(eps)
    x2, dy2 = _rows2d(x), _rows2d(dy)
    if dy2.shape != x2.shape:
        raise ValueError("dy must have the shape of x")
    m, n = x2.shape
    cidx = np.arange(n) if cols is None else np.asarray(cols)
    dg = np.zeros(len(cidx))
    db = np.zeros(len(cidx))
    for lo in range(0, m, chunk_rows):
        xc, dyc = _f64(x2[lo:lo + chunk_rows]), _f64(dy2[lo:lo + chunk_rows])
        mu, r = _stats(xc, eps)
        xhat = (xc[:, cidx] - mu[:, None]) * r[:, None]
        dyc = dyc[:, cidx]
        dg += np.sum(dyc * xhat, axis=0)
        db += np.sum(dyc, axis=0)
    return dg, db


def golden_ln_backward(dy, x, gamma, eps=DEFAULT_EPS, chunk_rows=CHUNK_ROWS):
    """Returns ``(dx, dgamma, dbeta)`` in float64 over all rows."""
    dx = golden_ln_dx(dy, x, gamma, eps, chunk_rows=chunk_rows)
    dg, db = golden_ln_param_grads(dy, x, eps, chunk_rows=chunk_rows)
    return dx, dg, db


def ln_param_condition(dy, x, eps, col):
    """Condition numbers ``sum|term| / |sum term|`` of the dgamma and dbeta
    column sums of column ``col`` (inf when a sum is exactly zero)."""
    x2, dy2 = _rows2d(x), _rows2d(dy)
    xc = _f64(x2)
    mu, r = _stats(xc, eps)
    tg = _f64(dy2[:, col]) * (xc[:, col] - mu) * r
    tb = _f64(dy2[:, col])

    def cond(t):
        s = abs(np.sum(t))
        return float(np.sum(np.abs(t)) / s) if s > 0 else float("inf")
    return cond(tg), cond(tb)


# ---- same-dtype reference (float32 intermediates, PyTorch CPU) -------------

def _t32(t):
    return _rows2d(t.detach().to("cpu")).float()


def reference_ln_forward(x, gamma, beta=None, eps=DEFAULT_EPS):
    """Returns ``(y, mean, rstd)``: y in x's dtype, mean and rstd float32."""
    xf = _t32(x)
    g = gamma.detach().to("cpu").float().reshape(-1)
    mean = xf.mean(-1, keepdim=True)
    d = xf - mean
    r = torch.rsqrt(d.square().mean(-1, keepdim=True) + eps)
    y = d * r * g
    if beta is not None:
        y = y + beta.detach().to("cpu").float().reshape(-1)
    return y.to(x.dtype), mean.squeeze(-1), r.squeeze(-1)


def reference_ln_backward(dy, x, gamma, eps=DEFAULT_EPS):
    """Explicit float32 backward.  Returns ``(dx, dgamma, dbeta)``: dx in x's
    dtype, the parameter gradients float32 sums over rows."""
    xf, dyf = _t32(x), _t32(dy)
    g = gamma.detach().to("cpu").float().reshape(-1)
    mean = xf.mean(-1, keepdim=True)
    d = xf - mean
    r = torch.rsqrt(d.square().mean(-1, keepdim=True) + eps)
    xhat = d * r
    u = dyf * g
    dx = r * (u - u.mean(-1, keepdim=True) - xhat * (u * xhat).mean(-1, keepdim=True))
    return dx.to(x.dtype), (dyf * xhat).sum(0), dyf.sum(0)


def reference_ln_param_grads(dy, x, eps=DEFAULT_EPS, cols=None):
    """dgamma and dbeta of ``reference_ln_backward`` for some columns only
    (same float32 operations, restricted to the columns ``cols``)."""
    xf, dyf = _t32(x), _t32(dy)
    mean = xf.mean(-1, keepdim=True)
    d = xf - mean
    r = torch.rsqrt(d.square().mean(-1, keepdim=True) + eps)
    xhat = d * r
    if cols is not None:
        idx = torch.as_tensor(cols, dtype=torch.long)
        xhat, dyf = xhat[:, idx], dyf[:, idx]
    return (dyf * xhat).sum(0), dyf.sum(0)


# ---- inputs of the fallback analysis (oracle.fallback) for dx --------------

def reference_ln_dx_reordered(dy, x, gamma, eps=DEFAULT_EPS):
    """dx of ``reference_ln_backward`` in a second legal float32 order: every
    row sum taken over the columns back to front, and r distributed over the
    three terms (r*u - r*mean(u) - (r*xhat)*mean(u*xhat)).  Returns dx in x's
    dtype."""
    xf, dyf = _t32(x), _t32(dy)
    g = gamma.detach().to("cpu").float().reshape(-1)
    n = xf.shape[-1]

    def rsum(t):
        return torch.flip(t, dims=[-1]).sum(-1, keepdim=True)

    mean = rsum(xf) / n
    d = xf - mean
    r = torch.rsqrt(rsum(d * d) / n + eps)
    xhat = d * r
    u = dyf * g
    dx = r * u - r * (rsum(u) / n) - (r * xhat) * (rsum(u * xhat) / n)
    return dx.to(x.dtype)


def ln_dx_magnitude(dy, x, gamma, eps=DEFAULT_EPS):
    """Per element, the magnitudes of the terms dx adds, in float64:
    r*(|u_ij| + mean_j|u_ij| + |xhat_ij| * mean_j|u_ij*xhat_ij|) -- the
    numerator of each element's condition number."""
    xd = _f64(x)
    xd = xd.reshape(-1, xd.shape[-1])
    ud = _f64(dy).reshape(xd.shape) * _vec(gamma, xd.shape[-1], "gamma")
    mu = xd.mean(-1, keepdims=True)
    d = xd - mu
    r = 1.0 / np.sqrt((d * d).mean(-1, keepdims=True) + eps)
    xh = d * r
    return r * (np.abs(ud) + np.abs(ud).mean(-1, keepdims=True)
                + np.abs(xh) * np.abs(ud * xh).mean(-1, keepdims=True))


def reference_ln_param_terms(dy, x, eps=DEFAULT_EPS):
    """The float32 per-row contributions the parameter gradients sum over the
    rows: ``(dy*xhat, dy)``, each [M, N], with the reference's xhat."""
    xf, dyf = _t32(x), _t32(dy)
    mean = xf.mean(-1, keepdim=True)
    d = xf - mean
    r = torch.rsqrt(d.square().mean(-1, keepdim=True) + eps)
    return dyf * (d * r), dyf
