"""Pins of the same-dtype float32 reference (oracle/reference.py).

The reference sets every gate's threshold (threshold = 2 * reference_error +
rounding floor), so it must itself be right.  It is pinned here, on the CPU,
to facts outside it:

* the printed worked values of the page "Check an AI model calculation before
  accelerating it" (tests/golden/worked_examples.json), to the printed
  digits;
* the float64 golden (itself pinned in test_oracle_pins.py), within a bound
  derived from float32 arithmetic: every product and quotient rounds once
  (relative error at most u = 2^-24) and a sum of n terms in any order is
  off by at most (n - 1) * u * sum|terms| to first order;
* for ``reference_dgamma`` (the column-restricted dgamma the sampled
  full-size gates use): equality with the columns of ``reference_backward``'s
  dgamma, and the golden's column sums within the bound above.

Planted mistakes in CPU copies of ``reference_dgamma`` (r dropped, a mean
instead of a sum, columns off by one, r from the selected columns only) each
fail the golden pin.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import golden, reference

HERE = os.path.dirname(os.path.abspath(__file__))
FIX = json.load(open(os.path.join(HERE, "golden", "worked_examples.json")))
EPS = 1e-6
U32 = 2.0 ** -24


def _inputs(M, N, seed, dtype=torch.float32):
    g = np.random.Generator(np.random.PCG64(seed))
    x = torch.from_numpy(g.standard_normal((M, N), dtype=np.float32)).to(dtype)
    w = torch.from_numpy(g.uniform(0.5, 1.5, N).astype(np.float32)).to(dtype)
    dy = torch.from_numpy(g.standard_normal((M, N), dtype=np.float32)).to(dtype)
    return x, w, dy


def _dgamma_bound(dy, x, M, N):
    """First-order float32 error bound of a column sum of dy*(x*r) over M rows,
    r carrying its own row-sum error (N terms) and a few roundings."""
    xd, dyd = x.double().numpy(), dy.double().numpy()
    r = 1.0 / np.sqrt((xd * xd).mean(-1, keepdims=True) + EPS)
    mag = np.abs(dyd * xd * r).sum(0)
    return 2.0 * (M + N + 8) * U32 * mag


def _printed_close(value, printed, decimals):
    """Equal to a value printed with `decimals` decimals: within half a unit of
    the last printed digit, plus float32 rounding of the value itself."""
    return abs(value - printed) <= 0.5 * 10.0 ** -decimals + 4 * U32 * abs(printed)


def test_worked_example_forward_matches_printed_values():
    for name in ("two_values", "two_values_gamma"):
        c = FIX[name]
        x = torch.tensor([c["x"]], dtype=torch.float32)
        w = torch.tensor(c["gamma"], dtype=torch.float32)
        y, r = reference.reference_forward(x, w, c["eps"])
        for got, want in zip(y[0].tolist(), c["printed"]["y"]):
            assert _printed_close(got, want, c["printed_decimals"]), (name, got, want)
        if "r" in c["printed"]:
            assert _printed_close(float(r[0]), c["printed"]["r"], c["printed_decimals"])


def test_worked_example_backward_matches_printed_values():
    c = FIX["dx_example"]
    x = torch.tensor([c["x"]], dtype=torch.float32)
    w = torch.tensor(c["gamma"], dtype=torch.float32)
    dy = torch.tensor([c["dy"]], dtype=torch.float32)
    dx, dg = reference.reference_backward(dy, x, w, c["eps"])
    for got, want in zip(dx[0].tolist(), c["printed"]["dx"]):
        assert _printed_close(got, want, c["printed_decimals"]), (got, want)
    # dgamma at M = 1 is that row's dy*x*r (derived from the page's definition,
    # not printed): [0.848528..., 2.262742...] with r from the golden.
    _, r_g = golden.golden_forward(x.numpy(), w.numpy(), c["eps"])
    want = np.asarray(c["dy"]) * np.asarray(c["x"]) * r_g[0]
    assert np.allclose(dg.double().numpy(), want, rtol=8 * U32, atol=0)
    assert np.allclose(reference.reference_dgamma(dy, x, c["eps"]).double().numpy(), want,
                       rtol=8 * U32, atol=0)


@pytest.mark.parametrize("M,N,dtype", [(257, 96, torch.float32), (300, 130, torch.bfloat16),
                                       (64, 1024, torch.float16)])
def test_reference_backward_dgamma_against_golden(M, N, dtype):
    x, w, dy = _inputs(M, N, 11, dtype)
    _, dg = reference.reference_backward(dy, x, w, EPS)
    dg_g = golden.golden_dgamma(dy, x, EPS)
    err = np.abs(dg.double().numpy() - dg_g)
    assert np.all(err <= _dgamma_bound(dy, x, M, N))


@pytest.mark.parametrize("M,N,dtype", [(257, 96, torch.float32), (300, 130, torch.bfloat16),
                                       (64, 1024, torch.float16)])
def test_reference_dgamma_columns_equal_full_backward(M, N, dtype):
    x, w, dy = _inputs(M, N, 12, dtype)
    _, dg = reference.reference_backward(dy, x, w, EPS)
    cols = [0, 1, N // 3, N // 2 + 1, N - 2, N - 1]
    sub = reference.reference_dgamma(dy, x, EPS, cols=cols)
    assert torch.equal(sub, dg[cols])
    assert torch.equal(reference.reference_dgamma(dy, x, EPS), dg)


# ---- planted mistakes in copies of reference_dgamma ------------------------

def _mut_no_r(dy, x, eps, cols):
    xf, dyf = x.float(), dy.float()
    return (dyf * xf).sum(0)[cols]


def _mut_mean(dy, x, eps, cols):
    xf, dyf = x.float(), dy.float()
    r = torch.rsqrt((xf * xf).sum(-1, keepdim=True) / xf.shape[-1] + eps)
    return (dyf * xf * r).mean(0)[cols]


def _mut_cols_shifted(dy, x, eps, cols):
    xf, dyf = x.float(), dy.float()
    r = torch.rsqrt((xf * xf).sum(-1, keepdim=True) / xf.shape[-1] + eps)
    shifted = [(c + 1) % xf.shape[-1] for c in cols]
    return (dyf * xf * r).sum(0)[shifted]


def _mut_r_from_selected_cols(dy, x, eps, cols):
    xf, dyf = x.float()[:, cols], dy.float()[:, cols]
    r = torch.rsqrt((xf * xf).sum(-1, keepdim=True) / xf.shape[-1] + eps)
    return (dyf * xf * r).sum(0)


def _golden_pin(impl, M=257, N=96):
    x, _, dy = _inputs(M, N, 13)
    cols = [0, 5, 17, 48, 95]
    got = impl(dy, x, EPS, cols).double().numpy()
    want = golden.golden_dgamma(dy, x, EPS, cols=cols)
    return bool(np.all(np.abs(got - want) <= _dgamma_bound(dy, x, M, N)[cols]))


def test_reference_dgamma_holds_the_golden_pin():
    assert _golden_pin(lambda dy, x, eps, cols: reference.reference_dgamma(dy, x, eps, cols))


@pytest.mark.parametrize("mutant", [_mut_no_r, _mut_mean, _mut_cols_shifted,
                                    _mut_r_from_selected_cols])
def test_golden_pin_catches_planted_mistake(mutant):
    assert not _golden_pin(mutant)


def test_reference_forward_and_dx_against_golden():
    """y and dx of the reference within a float32 bound of the golden (rows of
    N = 96: r carries about N roundings; y is x*r*g; dx's two terms are bounded
    by |r*u| + |x*r^3*c|)."""
    M, N = 33, 96
    x, w, dy = _inputs(M, N, 14)
    y, r = reference.reference_forward(x, w, EPS)
    dx, _ = reference.reference_backward(dy, x, w, EPS)
    y_g, r_g = golden.golden_forward(x, w, EPS)
    dx_g = golden.golden_dx(dy, x, w, EPS)
    k = (N + 8) * U32
    assert np.all(np.abs(r.double().numpy() - r_g) <= k * r_g)
    assert np.all(np.abs(y.double().numpy() - y_g) <= 2 * k * np.abs(y_g) + 1e-30)
    xd, dyd, wd = x.double().numpy(), dy.double().numpy(), w.double().numpy()
    rr = r_g[:, None]
    c = (dyd * wd * xd).mean(-1, keepdims=True)
    scale = np.abs(rr * dyd * wd) + np.abs(xd * rr ** 3 * c) + rr ** 3 * np.abs(xd) * \
        (np.abs(dyd * wd * xd).mean(-1, keepdims=True))
    assert np.all(np.abs(dx.double().numpy() - dx_g) <= 2 * k * scale)
