"""Float64 golden RMSNorm forward and backward (test infrastructure only).

The golden is the plain definition of the operation, evaluated in float64 with
NumPy on the same low-precision inputs the kernel sees, promoted losslessly to
float64 (torchtitan kernel-numerics-verifier page, section "核心方法": one
low-precision input set, promoted without loss for the golden; the golden
keeps its float64 result and is never cast back).

Definitions followed (page "Check an AI model calculation before accelerating
it", partitech):

* section "Problem and reference formula": per row,
  ``r = 1 / sqrt(mean(x**2) + eps)`` and ``y = x * r * gamma``; eps sits inside
  the square root and keeps an all-zero row finite.
* section "N and BLOCK: two sizes you must never confuse": the mean divides by
  the logical row length N.
* section "Input backward pass: keep the right N" and "Where does the cube of r
  come from?": with ``u = dy * gamma``,
  ``dx = r * u - x * r**3 * mean(u * x)`` (mean over the N columns of the row).
* section "A sum is not an average": ``dgamma = sum over rows of dy * x * r``
  (no division by M).
* torchtitan page, section "仓库实例 OffsetRMSNorm": in offset mode the weight
  is applied as ``(1 + w)``, the 1 being added after promotion.  Because
  d(1 + w)/dw = 1, dgamma has the same expression in both modes (chain rule).

Work is chunked over rows so that large inputs never need a full float64 copy.
Inputs may be NumPy arrays or PyTorch CPU tensors of any floating dtype
(bfloat16 included); leading dimensions are flattened into rows.
"""
from __future__ import annotations

import numpy as np

DEFAULT_EPS = 1e-6
CHUNK_ROWS = 4096


def _rows2d(a):
    """View ``a`` as [M, N] (leading dims flattened into rows)."""
    if a.ndim == 1:
        return a.reshape(1, -1)
    return a.reshape(-1, a.shape[-1])


def _f64(a):
    """Lossless promotion of a NumPy array or a torch tensor to float64."""
    if hasattr(a, "detach"):  # torch tensor: bfloat16 has no NumPy dtype
        return a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def _weight(weight, offset):
    g = _f64(weight).reshape(-1)
    if offset:
        g = 1.0 + g
    return g


def _check_eps(eps):
    if not (np.isfinite(eps) and eps > 0):
        raise ValueError("eps must be finite and positive")


def _row_rstd(xc, eps):
    """r = 1/sqrt(mean(x^2) + eps) for each row of a float64 chunk."""
    n = xc.shape[1]
    ms = np.sum(xc * xc, axis=1) / n
    return 1.0 / np.sqrt(ms + eps)


def golden_rstd(x, eps=DEFAULT_EPS, rows=None, chunk_rows=CHUNK_ROWS):
    """Per-row inverse RMS r (float64, shape [M] or [len(rows)])."""
    _check_eps(eps)
    x2 = _rows2d(x)
    idx = np.arange(x2.shape[0]) if rows is None else np.asarray(rows)
    out = np.empty(len(idx), dtype=np.float64)
    for lo in range(0, len(idx), chunk_rows):
        sel = idx[lo:lo + chunk_rows]
        out[lo:lo + len(sel)] = _row_rstd(_f64(x2[sel]), eps)
    return out


def golden_forward(x, weight, eps=DEFAULT_EPS, offset=False, rows=None,
                   chunk_rows=CHUNK_ROWS):
    """Golden forward.  Returns ``(y, r)``: y float64 [R, N], r float64 [R].

    ``rows`` (optional) selects a subset of rows; R = M when it is None.
    """
    _check_eps(eps)
    x2 = _rows2d(x)
    g = _weight(weight, offset)
    if g.shape[0] != x2.shape[1]:
        raise ValueError("weight length must equal the row length N")
    idx = np.arange(x2.shape[0]) if rows is None else np.asarray(rows)
    y = np.empty((len(idx), x2.shape[1]), dtype=np.float64)
    r = np.empty(len(idx), dtype=np.float64)
    for lo in range(0, len(idx), chunk_rows):
        sel = idx[lo:lo + chunk_rows]
        xc = _f64(x2[sel])
        rc = _row_rstd(xc, eps)
        y[lo:lo + len(sel)] = xc * rc[:, None] * g[None, :]
        r[lo:lo + len(sel)] = rc
    return y, r


def golden_dx(dy, x, weight, eps=DEFAULT_EPS, offset=False, rows=None,
              chunk_rows=CHUNK_ROWS):
    """Golden input gradient dx (float64, [R, N]) for all or selected rows."""
    _check_eps(eps)
    x2 = _rows2d(x)
    dy2 = _rows2d(dy)
    if dy2.shape != x2.shape:
        raise ValueError("dy must have the shape of x")
    g = _weight(weight, offset)
    n = x2.shape[1]
    idx = np.arange(x2.shape[0]) if rows is None else np.asarray(rows)
    dx = np.empty((len(idx), n), dtype=np.float64)
    for lo in range(0, len(idx), chunk_rows):
        sel = idx[lo:lo + chunk_rows]
        xc = _f64(x2[sel])
        dyc = _f64(dy2[sel])
        rc = _row_rstd(xc, eps)[:, None]
        u = dyc * g[None, :]
        c = np.sum(u * xc, axis=1, keepdims=True) / n
        dx[lo:lo + len(sel)] = rc * u - xc * rc ** 3 * c
    return dx


def golden_dgamma(dy, x, eps=DEFAULT_EPS, cols=None, chunk_rows=CHUNK_ROWS):
    """Golden weight gradient: the column sum over ALL rows of dy * x * r.

    ``cols`` (optional) restricts the output to some columns; r still comes
    from whole rows.  The weight itself does not enter (in either mode).
    """
    _check_eps(eps)
    x2 = _rows2d(x)
    dy2 = _rows2d(dy)
    if dy2.shape != x2.shape:
        raise ValueError("dy must have the shape of x")
    m, n = x2.shape
    cidx = np.arange(n) if cols is None else np.asarray(cols)
    acc = np.zeros(len(cidx), dtype=np.float64)
    for lo in range(0, m, chunk_rows):
        xc = _f64(x2[lo:lo + chunk_rows])
        rc = _row_rstd(xc, eps)
        if cols is not None:
            xc = xc[:, cidx]
        dyc = _f64(dy2[lo:lo + chunk_rows])
        if cols is not None:
            dyc = dyc[:, cidx]
        acc += np.sum(dyc * xc * rc[:, None], axis=0)
    return acc


def golden_backward(dy, x, weight, eps=DEFAULT_EPS, offset=False,
                    chunk_rows=CHUNK_ROWS):
    """Golden backward over all rows.  Returns ``(dx, dgamma)`` in float64."""
    dx = golden_dx(dy, x, weight, eps, offset, chunk_rows=chunk_rows)
    dgamma = golden_dgamma(dy, x, eps, chunk_rows=chunk_rows)
    return dx, dgamma


def dgamma_condition(dy, x, eps, col):
    """Per-element condition number of one dgamma column sum.

    ``sum|term| / |sum term|`` over the float64 per-row terms dy*x*r of column
    ``col`` (torchtitan page, section on reductions: the condition number
    explains a large error through cancellation; it does not prove a result
    right).  Returns inf when the column sums to exactly zero.
    """
    x2 = _rows2d(x)
    dy2 = _rows2d(dy)
    r = golden_rstd(x2, eps)
    terms = _f64(dy2[:, col]) * _f64(x2[:, col]) * r
    s = abs(np.sum(terms))
    return float(np.sum(np.abs(terms)) / s) if s > 0 else float("inf")
