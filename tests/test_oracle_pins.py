"""Pins of the float64 golden to facts fixed outside the oracle itself.

Every check is written as a function of the implementation under test, so the
same checks are run twice: on the golden (must pass) and on deliberately
broken CPU variants of it, each carrying one plausible mistake (must fail).
That shows each pin can actually catch the mistake it is meant for.

Sources: the printed values of the page "Check an AI model calculation before
accelerating it" (stored in tests/golden/worked_examples.json with their
sections), closed forms and invariants that follow from its definitions,
central differences (its section "PyTorch reference: the numerical oracle"
estimates slopes this way), and PyTorch's own float64 ``rms_norm`` with
autograd as an independent library implementation.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import golden

HERE = os.path.dirname(os.path.abspath(__file__))
FIX = json.load(open(os.path.join(HERE, "golden", "worked_examples.json")))
EPS = 1e-6


# ----------------------------------------------------------------------------
# Implementations under test: the golden, and CPU variants with one mistake.
# ----------------------------------------------------------------------------
class Impl:
    """forward(x, g, eps, offset) -> (y, r); dx(dy, x, g, eps, offset);
    dgamma(dy, x, eps)"""

    def __init__(self, name, forward, dx, dgamma):
        self.name, self.forward, self.dx, self.dgamma = name, forward, dx, dgamma


GOLDEN = Impl("golden",
              lambda x, g, eps=EPS, offset=False: golden.golden_forward(x, g, eps, offset),
              lambda dy, x, g, eps=EPS, offset=False: golden.golden_dx(dy, x, g, eps, offset),
              lambda dy, x, eps=EPS: golden.golden_dgamma(dy, x, eps))


def _mut_forward(denominator=None, eps_outside=False, offset_dropped=False):
    def fwd(x, g, eps=EPS, offset=False):
        x = np.atleast_2d(np.asarray(x, dtype=np.float64))
        g = np.asarray(g, dtype=np.float64)
        if offset and not offset_dropped:
            g = 1.0 + g
        n = x.shape[1]
        d = n if denominator is None else denominator(n)
        ms = np.sum(x * x, axis=1) / d
        r = 1.0 / (np.sqrt(ms) + eps) if eps_outside else 1.0 / np.sqrt(ms + eps)
        return x * r[:, None] * g[None, :], r
    return fwd


def _mut_dx(power=3, denominator=None, sign=-1.0):
    def dx(dy, x, g, eps=EPS, offset=False):
        x = np.atleast_2d(np.asarray(x, dtype=np.float64))
        dy = np.atleast_2d(np.asarray(dy, dtype=np.float64))
        g = np.asarray(g, dtype=np.float64)
        if offset:
            g = 1.0 + g
        n = x.shape[1]
        d = n if denominator is None else denominator(n)
        r = (1.0 / np.sqrt(np.sum(x * x, axis=1) / n + eps))[:, None]
        u = dy * g
        c = np.sum(u * x, axis=1, keepdims=True) / d
        return r * u + sign * x * r ** power * c
    return dx


def _mut_dgamma(mean=False, drop_r=False):
    def dgamma(dy, x, eps=EPS):
        x = np.atleast_2d(np.asarray(x, dtype=np.float64))
        dy = np.atleast_2d(np.asarray(dy, dtype=np.float64))
        r = 1.0 / np.sqrt(np.sum(x * x, axis=1) / x.shape[1] + eps)
        t = dy * x * (1.0 if drop_r else r[:, None])
        return t.mean(0) if mean else t.sum(0)
    return dgamma


def _next_pow2(n):
    return 1 << (n - 1).bit_length()


MUTANTS = {
    "padded_denominator": Impl("padded_denominator",
                               _mut_forward(denominator=_next_pow2),
                               _mut_dx(denominator=_next_pow2), GOLDEN.dgamma),
    "eps_outside_sqrt": Impl("eps_outside_sqrt", _mut_forward(eps_outside=True),
                             GOLDEN.dx, GOLDEN.dgamma),
    "offset_dropped": Impl("offset_dropped", _mut_forward(offset_dropped=True),
                           GOLDEN.dx, GOLDEN.dgamma),
    "r_squared_in_dx": Impl("r_squared_in_dx", GOLDEN.forward, _mut_dx(power=2),
                            GOLDEN.dgamma),
    "sign_flip_in_dx": Impl("sign_flip_in_dx", GOLDEN.forward, _mut_dx(sign=+1.0),
                            GOLDEN.dgamma),
    "dgamma_mean": Impl("dgamma_mean", GOLDEN.forward, GOLDEN.dx,
                        _mut_dgamma(mean=True)),
    "dgamma_without_r": Impl("dgamma_without_r", GOLDEN.forward, GOLDEN.dx,
                             _mut_dgamma(drop_r=True)),
}


# ----------------------------------------------------------------------------
# The pins, each a function of an implementation; True when it holds.
# ----------------------------------------------------------------------------
def _close_printed(value, printed, decimals):
    return abs(value - printed) <= 0.5 * 10.0 ** (-decimals) + 1e-12


def pin_two_values(impl):
    f = FIX["two_values"]
    y, r = impl.forward(np.array([f["x"]]), np.array(f["gamma"]), f["eps"])
    p, d = f["printed"], f["printed_decimals"]
    ok = all(_close_printed(a, b, d) for a, b in zip(y[0], p["y"]))
    ok &= _close_printed(r[0], p["r"], d)
    ok &= _close_printed(1.0 / r[0], p["stabilized_denominator"], d)
    # the mean of squares is recovered from r: 1/r^2 - eps
    ok &= abs(1.0 / r[0] ** 2 - f["eps"] - p["mean_of_squares"]) < 1e-9
    return bool(ok)


def pin_two_values_gamma(impl):
    f = FIX["two_values_gamma"]
    y, _ = impl.forward(np.array([f["x"]]), np.array(f["gamma"]), f["eps"])
    return all(_close_printed(a, b, f["printed_decimals"])
               for a, b in zip(y[0], f["printed"]["y"]))


def pin_dx_example(impl):
    f = FIX["dx_example"]
    dx = impl.dx(np.array([f["dy"]]), np.array([f["x"]]), np.array(f["gamma"]),
                 f["eps"])
    return all(_close_printed(a, b, f["printed_decimals"])
               for a, b in zip(dx[0], f["printed"]["dx"]))


def pin_dgamma_sum_table(impl):
    """Rows whose contributions dy*x*r are the page's table sum to [4, 6]."""
    f = FIX["dgamma_sum_table"]
    c = np.array(f["contributions"])
    x = np.array([[1.0, 2.0], [3.0, 4.0]])
    _, r = GOLDEN.forward(x, np.ones(2), EPS)  # r from the (pinned) forward
    dy = c / (x * r[:, None])
    dg = impl.dgamma(dy, x, EPS)
    return bool(np.allclose(dg, f["printed"]["sum"], rtol=0, atol=1e-12))


def pin_dgamma_m1_vs_m17(impl):
    """M=1: dgamma_j = dy_j * y_j / gamma_j (same r as the forward);
    M=17 copies of that row: exactly 17 times as much (a sum, not a mean)."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 9))
    dy = rng.standard_normal((1, 9))
    g = rng.uniform(0.5, 1.5, 9)
    y, _ = GOLDEN.forward(x, g, EPS)
    d1 = impl.dgamma(dy, x, EPS)
    d17 = impl.dgamma(np.repeat(dy, 17, 0), np.repeat(x, 17, 0), EPS)
    ok = np.allclose(d1, (dy * y / g)[0], rtol=1e-13, atol=0)
    ok &= np.allclose(d17, 17.0 * d1, rtol=1e-13, atol=0)
    return bool(ok)


def pin_logical_n(impl):
    f = FIX["logical_n_exercise"]
    n, p, dec = f["n"], f["printed"], f["printed_decimals"]
    y, r = impl.forward(np.ones((1, n)), np.ones(n), f["eps"])
    ok = _close_printed(1.0 / r[0], p["denominator_correct"], dec["denominator_correct"])
    ok &= bool(np.all(np.abs(y - p["output_correct"]) <= 0.5e-7 + 1e-12))
    # the page's [1,1,1] row: the mean of squares is 1, not 0.75
    _, r3 = impl.forward(np.ones((1, 3)), np.ones(3), EPS)
    ok &= abs(1.0 / r3[0] ** 2 - EPS - 1.0) < 1e-9
    return bool(ok)


def pin_zero_row(impl):
    """An all-zero row: y = 0 and r = eps^-1/2; dx = r*dy*gamma; no dgamma."""
    n = 5
    g = np.array([0.5, 1.0, 1.5, 2.0, 2.5])
    dy = np.arange(1.0, n + 1.0)[None, :]
    y, r = impl.forward(np.zeros((1, n)), g, EPS)
    dx = impl.dx(dy, np.zeros((1, n)), g, EPS)
    dg = impl.dgamma(dy, np.zeros((1, n)), EPS)
    ok = bool(np.all(y == 0.0)) and abs(r[0] - 1000.0) < 1e-9
    ok &= bool(np.allclose(dx[0], r[0] * dy[0] * g, rtol=1e-14, atol=0))
    ok &= bool(np.all(dg == 0.0))
    return ok


def pin_mean_square_identity(impl):
    """mean((y/g)^2) = ms/(ms+eps), with ms measured here from x."""
    rng = np.random.default_rng(5)
    for n in (7, 257):
        x = rng.standard_normal((6, n)) * np.array([1, 1e-3, 3e-4, 1e2, 1, 0.1])[:, None]
        g = rng.uniform(0.5, 1.5, n)
        y, _ = impl.forward(x, g, EPS)
        ms = np.mean(x * x, axis=1)
        lhs = np.mean((y / g) ** 2, axis=1)
        if not np.allclose(lhs, ms / (ms + EPS), rtol=1e-12, atol=0):
            return False
    return True


def pin_scale_invariance(impl):
    """y(a*x) = y(x) only while a^2*ms >> eps: exact up to eps/ms at a=1e3,
    broken at a=1e-3 where a^2*ms ~ eps (eps sits inside the square root)."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((4, 64))
    g = rng.uniform(0.5, 1.5, 64)
    y, _ = impl.forward(x, g, EPS)
    y_up, _ = impl.forward(1e3 * x, g, EPS)
    y_dn, _ = impl.forward(1e-3 * x, g, EPS)
    ms = np.mean(x * x, axis=1, keepdims=True)
    rel_up = np.max(np.abs(y_up / y - 1.0) / (EPS / ms))
    rel_dn = np.max(np.abs(y_dn / y - 1.0))
    return bool(rel_up <= 0.51 and rel_dn > 0.1)


def pin_dx_orthogonal_to_x(impl):
    """sum_j x_j dx_j = r*N*c*eps/(ms+eps): ~0 for eps << ms (y does not
    change when x is scaled), and of that size when eps is not small."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((5, 33))
    dy = rng.standard_normal((5, 33))
    g = rng.uniform(0.5, 1.5, 33)
    for eps in (EPS, 0.7):
        dx = impl.dx(dy, x, g, eps)
        ms = np.mean(x * x, axis=1)
        r = 1.0 / np.sqrt(ms + eps)
        c = np.mean(dy * g * x, axis=1)
        lhs = np.sum(x * dx, axis=1)
        rhs = r * x.shape[1] * c * eps / (ms + eps)
        scale = np.sum(np.abs(x * dx), axis=1)
        if not np.all(np.abs(lhs - rhs) <= 1e-12 * scale):
            return False
    return True


def pin_offset_equals_gamma(impl):
    """Offset weight w behaves as gamma = 1 + w formed in float64."""
    rng = np.random.default_rng(13)
    x = rng.standard_normal((3, 40))
    dy = rng.standard_normal((3, 40))
    w = rng.standard_normal(40) * 0.02
    y_o, r_o = impl.forward(x, w, EPS, True)
    y_g, r_g = impl.forward(x, 1.0 + w, EPS, False)
    dx_o = impl.dx(dy, x, w, EPS, True)
    dx_g = impl.dx(dy, x, 1.0 + w, EPS, False)
    return bool(np.array_equal(y_o, y_g) and np.array_equal(r_o, r_g)
                and np.array_equal(dx_o, dx_g)
                and not np.allclose(y_o, impl.forward(x, w, EPS, False)[0]))


def _loss(impl, x, g, dy, offset=False):
    y, _ = impl.forward(x, g, EPS, offset)
    return float(np.sum(dy * y))


def pin_central_differences(impl):
    """dx and dgamma equal the central-difference slope of L = sum(dy*y)."""
    rng = np.random.default_rng(17)
    m, n, h = 3, 7, 1e-6
    x = rng.standard_normal((m, n))
    dy = rng.standard_normal((m, n))
    for offset in (False, True):
        g = rng.standard_normal(n) * 0.02 if offset else rng.uniform(0.5, 1.5, n)
        num_dx = np.zeros_like(x)
        for i in range(m):
            for j in range(n):
                xp, xm = x.copy(), x.copy()
                xp[i, j] += h
                xm[i, j] -= h
                num_dx[i, j] = (_loss(impl, xp, g, dy, offset)
                                - _loss(impl, xm, g, dy, offset)) / (2 * h)
        num_dg = np.zeros(n)
        for j in range(n):
            gp, gm = g.copy(), g.copy()
            gp[j] += h
            gm[j] -= h
            num_dg[j] = (_loss(impl, x, gp, dy, offset)
                         - _loss(impl, x, gm, dy, offset)) / (2 * h)
        if not np.allclose(impl.dx(dy, x, g, EPS, offset), num_dx, rtol=0, atol=1e-8):
            return False
        if not np.allclose(impl.dgamma(dy, x, EPS), num_dg, rtol=0, atol=1e-8):
            return False
    return True


def pin_torch_rms_norm(impl):
    """Agreement with torch.nn.functional.rms_norm and its autograd (fp64)."""
    rng = np.random.default_rng(19)
    for n in (2, 129, 1024):
        x = rng.standard_normal((5, n))
        dy = rng.standard_normal((5, n))
        g = rng.uniform(0.5, 1.5, n)
        xt = torch.tensor(x, requires_grad=True)
        gt = torch.tensor(g, requires_grad=True)
        yt = torch.nn.functional.rms_norm(xt, (n,), gt, EPS)
        dxt, dgt = torch.autograd.grad(yt, (xt, gt), torch.tensor(dy))
        y, _ = impl.forward(x, g, EPS)
        if not np.allclose(y, yt.detach().numpy(), rtol=1e-13, atol=1e-15):
            return False
        if not np.allclose(impl.dx(dy, x, g, EPS), dxt.numpy(), rtol=1e-11, atol=1e-13):
            return False
        if not np.allclose(impl.dgamma(dy, x, EPS), dgt.numpy(), rtol=1e-11, atol=1e-13):
            return False
    return True


PINS = {
    "two_values": pin_two_values,
    "two_values_gamma": pin_two_values_gamma,
    "dx_example": pin_dx_example,
    "dgamma_sum_table": pin_dgamma_sum_table,
    "dgamma_m1_vs_m17": pin_dgamma_m1_vs_m17,
    "logical_n": pin_logical_n,
    "zero_row": pin_zero_row,
    "mean_square_identity": pin_mean_square_identity,
    "scale_invariance": pin_scale_invariance,
    "dx_orthogonal_to_x": pin_dx_orthogonal_to_x,
    "offset_equals_gamma": pin_offset_equals_gamma,
    "central_differences": pin_central_differences,
    "torch_rms_norm": pin_torch_rms_norm,
}


@pytest.mark.parametrize("pin", sorted(PINS))
def test_golden_holds_pin(pin):
    assert PINS[pin](GOLDEN), f"golden fails pin {pin}"


# Which pins must catch which planted mistake (each mutant is caught by at
# least one pin; the listed ones are those that must fail).
CAUGHT_BY = {
    "padded_denominator": ["logical_n", "mean_square_identity", "torch_rms_norm"],
    "eps_outside_sqrt": ["two_values", "zero_row", "mean_square_identity", "torch_rms_norm"],
    "offset_dropped": ["offset_equals_gamma", "central_differences"],
    "r_squared_in_dx": ["dx_example", "dx_orthogonal_to_x", "central_differences",
                        "torch_rms_norm"],
    "sign_flip_in_dx": ["dx_example", "dx_orthogonal_to_x", "central_differences"],
    "dgamma_mean": ["dgamma_sum_table", "dgamma_m1_vs_m17"],
    "dgamma_without_r": ["dgamma_sum_table", "dgamma_m1_vs_m17", "central_differences",
                         "torch_rms_norm"],
}


@pytest.mark.parametrize("mutant,pin", [(m, p) for m, ps in sorted(CAUGHT_BY.items())
                                        for p in ps])
def test_pin_catches_planted_mistake(mutant, pin):
    assert not PINS[pin](MUTANTS[mutant]), f"pin {pin} misses mutant {mutant}"


def test_logical_n_printed_wrong_values_come_from_padded_block():
    """The page's 'incorrect division by BLOCK' column is what the padded
    mutant computes: the pin compares against the right column."""
    f = FIX["logical_n_exercise"]
    p, dec = f["printed"], f["printed_decimals"]
    y, r = MUTANTS["padded_denominator"].forward(np.ones((1, 257)), np.ones(257), EPS)
    assert _close_printed(1.0 / r[0], p["denominator_wrong"], dec["denominator_wrong"])
    assert _close_printed(y[0, 0], p["output_wrong"], dec["output_wrong"])
    assert abs((1.0 / r[0] ** 2 - EPS) - p["average_wrong"]) < 1e-9


# ----------------------------------------------------------------------------
# Golden plumbing: chunking, row/column subsets, dtypes and leading dims.
# ----------------------------------------------------------------------------
def test_chunking_and_subsets_agree():
    rng = np.random.default_rng(23)
    x = rng.standard_normal((37, 19))
    dy = rng.standard_normal((37, 19))
    g = rng.uniform(0.5, 1.5, 19)
    y, r = golden.golden_forward(x, g, EPS)
    y3, r3 = golden.golden_forward(x, g, EPS, chunk_rows=3)
    assert np.array_equal(y, y3) and np.array_equal(r, r3)
    rows = np.array([0, 5, 36, 17])
    ys, rs = golden.golden_forward(x, g, EPS, rows=rows, chunk_rows=2)
    assert np.array_equal(ys, y[rows]) and np.array_equal(rs, r[rows])
    assert np.array_equal(golden.golden_rstd(x, EPS, rows=rows), r[rows])
    dx = golden.golden_dx(dy, x, g, EPS)
    assert np.array_equal(golden.golden_dx(dy, x, g, EPS, rows=rows, chunk_rows=3), dx[rows])
    dg = golden.golden_dgamma(dy, x, EPS)
    dg3 = golden.golden_dgamma(dy, x, EPS, chunk_rows=3)
    assert np.allclose(dg, dg3, rtol=1e-14, atol=1e-15)
    cols = np.array([18, 0, 7])
    assert np.allclose(golden.golden_dgamma(dy, x, EPS, cols=cols, chunk_rows=4), dg[cols],
                       rtol=1e-14, atol=1e-15)


def test_torch_low_precision_inputs_are_promoted_losslessly():
    t = torch.tensor([[3.0, 4.0], [0.1, -7.25]]).to(torch.bfloat16)
    g = torch.tensor([1.0, 1.0]).to(torch.bfloat16)
    y, r = golden.golden_forward(t, g, EPS)
    x64 = t.double().numpy()
    y2, r2 = golden.golden_forward(x64, g.double().numpy(), EPS)
    assert np.array_equal(y, y2) and np.array_equal(r, r2)


def test_leading_dims_flatten_into_rows():
    rng = np.random.default_rng(29)
    x = rng.standard_normal((2, 3, 8))
    g = rng.uniform(0.5, 1.5, 8)
    y, r = golden.golden_forward(x, g, EPS)
    y2, r2 = golden.golden_forward(x.reshape(6, 8), g, EPS)
    assert np.array_equal(y, y2) and y.shape == (6, 8)


@pytest.mark.parametrize("bad", [0.0, -1e-6, float("nan"), float("inf")])
def test_bad_eps_rejected(bad):
    with pytest.raises(ValueError):
        golden.golden_forward(np.ones((1, 2)), np.ones(2), bad)


def test_condition_number_of_cancelling_column():
    x = np.array([[1.0, 1.0], [1.0, 1.0]])
    dy = np.array([[1.0, 2.0], [-1.0, 2.0]])
    assert golden.dgamma_condition(dy, x, EPS, 1) == pytest.approx(1.0)
    assert math.isinf(golden.dgamma_condition(dy, x, EPS, 0))
