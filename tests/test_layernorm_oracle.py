"""Pins of the float64 LayerNorm golden (oracle.layernorm) to facts fixed
outside it, run on the golden (must hold) and on CPU variants that each carry
one plausible mistake (must fail), as for the RMSNorm golden.

Sources: closed forms that follow from the definition of the page "PyTorch
torch.compile ... LayerNorm and RMSNorm", section 1.1 (mean and variance of
the row, weight and bias), invariants of that definition, central differences
of L = sum(dy * y), and PyTorch's own float64 ``layer_norm`` with autograd as
an independent library implementation.  The same-dtype reference is checked
against the golden.
"""
import numpy as np
import pytest
import torch

from oracle import layernorm as ln

EPS = 1e-6


class Impl:
    """forward(x, g, b, eps) -> (y, mean, rstd); dx(dy, x, g, eps);
    params(dy, x, eps) -> (dgamma, dbeta)"""

    def __init__(self, name, forward, dx, params):
        self.name, self.forward, self.dx, self.params = name, forward, dx, params


GOLDEN = Impl("golden",
              lambda x, g, b=None, eps=EPS: ln.golden_ln_forward(x, g, b, eps),
              lambda dy, x, g, eps=EPS: ln.golden_ln_dx(dy, x, g, eps),
              lambda dy, x, eps=EPS: ln.golden_ln_param_grads(dy, x, eps))


def _a(v):
    return np.atleast_2d(np.asarray(v, dtype=np.float64))


def _mut_stats(x, eps, unbiased=False, centred=True, eps_outside=False):
    n = x.shape[1]
    mu = x.mean(1) if centred else np.zeros(x.shape[0])
    d = x - mu[:, None]
    var = np.sum(d * d, axis=1) / (n - 1 if unbiased else n)
    r = 1.0 / (np.sqrt(var) + eps) if eps_outside else 1.0 / np.sqrt(var + eps)
    return mu, r


def _mut_forward(drop_beta=False, **kw):
    def fwd(x, g, b=None, eps=EPS):
        x = _a(x)
        g = np.asarray(g, dtype=np.float64)
        b = np.zeros(x.shape[1]) if (b is None or drop_beta) else np.asarray(b, dtype=np.float64)
        mu, r = _mut_stats(x, eps, **kw)
        return (x - mu[:, None]) * r[:, None] * g + b, mu, r
    return fwd


def _mut_dx(drop_mean_u=False, drop_xhat_term=False, **kw):
    def dx(dy, x, g, eps=EPS):
        x, dy = _a(x), _a(dy)
        g = np.asarray(g, dtype=np.float64)
        mu, r = _mut_stats(x, eps, **kw)
        xhat = (x - mu[:, None]) * r[:, None]
        u = dy * g
        t = u.copy()
        if not drop_mean_u:
            t -= u.mean(1, keepdims=True)
        if not drop_xhat_term:
            t -= xhat * (u * xhat).mean(1, keepdims=True)
        return r[:, None] * t
    return dx


def _mut_params(dbeta_mean=False, drop_r=False):
    def params(dy, x, eps=EPS):
        x, dy = _a(x), _a(dy)
        mu, r = _mut_stats(x, eps)
        xhat = (x - mu[:, None]) * (1.0 if drop_r else r[:, None])
        db = dy.mean(0) if dbeta_mean else dy.sum(0)
        return (dy * xhat).sum(0), db
    return params


MUTANTS = {
    "unbiased_variance": Impl("unbiased_variance", _mut_forward(unbiased=True),
                              _mut_dx(unbiased=True), GOLDEN.params),
    "not_centred": Impl("not_centred", _mut_forward(centred=False),
                        _mut_dx(centred=False), GOLDEN.params),
    "eps_outside_sqrt": Impl("eps_outside_sqrt", _mut_forward(eps_outside=True),
                             GOLDEN.dx, GOLDEN.params),
    "beta_dropped": Impl("beta_dropped", _mut_forward(drop_beta=True), GOLDEN.dx,
                         GOLDEN.params),
    "dx_without_mean_u": Impl("dx_without_mean_u", GOLDEN.forward,
                              _mut_dx(drop_mean_u=True), GOLDEN.params),
    "dx_without_xhat_term": Impl("dx_without_xhat_term", GOLDEN.forward,
                                 _mut_dx(drop_xhat_term=True), GOLDEN.params),
    "dbeta_mean": Impl("dbeta_mean", GOLDEN.forward, GOLDEN.dx, _mut_params(dbeta_mean=True)),
    "dgamma_without_r": Impl("dgamma_without_r", GOLDEN.forward, GOLDEN.dx,
                             _mut_params(drop_r=True)),
}


# ---- pins ---------------------------------------------------------------------

def pin_two_values(impl):
    """x = [3, 4]: mean 3.5, variance 1/4 (the squared half-distance), so
    y = [-r/2, r/2] * gamma + beta with r = 1/sqrt(1/4 + eps)."""
    r = 1.0 / np.sqrt(0.25 + EPS)
    y, mu, rs = impl.forward([[3.0, 4.0]], np.array([1.0, 1.0]), None, EPS)
    ok = np.allclose(y, [[-0.5 * r, 0.5 * r]], rtol=1e-15, atol=0) and \
        np.isclose(mu[0], 3.5, rtol=0, atol=0) and np.isclose(rs[0], r, rtol=1e-15, atol=0)
    y2, _, _ = impl.forward([[3.0, 4.0]], np.array([2.0, 0.5]), np.array([0.5, -0.25]), EPS)
    return bool(ok and np.allclose(y2, [[-r + 0.5, 0.25 * r - 0.25]], rtol=1e-15, atol=1e-16))


def pin_biased_variance(impl):
    """x = [0, 2, 0, 2]: the mean of squared deviations is 1 (divide by N)."""
    _, mu, r = impl.forward([[0.0, 2.0, 0.0, 2.0]], np.ones(4), None, EPS)
    return bool(mu[0] == 1.0 and np.isclose(r[0], 1.0 / np.sqrt(1.0 + EPS), rtol=1e-15))


def pin_constant_row(impl):
    """A constant row has zero variance: xhat = 0, so y = beta exactly,
    r = 1/sqrt(eps), and dx = r * (u - mean(u))."""
    n = 6
    rng = np.random.default_rng(3)
    g = rng.uniform(0.5, 1.5, n)
    b = rng.uniform(-0.5, 0.5, n)
    x = np.full((1, n), 0.75)
    dy = rng.standard_normal((1, n))
    y, mu, r = impl.forward(x, g, b, EPS)
    re = 1.0 / np.sqrt(EPS)
    u = dy * g
    dx = impl.dx(dy, x, g, EPS)
    return bool(np.array_equal(y, b[None, :]) and np.isclose(r[0], re, rtol=1e-15)
                and np.allclose(dx, re * (u - u.mean()), rtol=1e-13, atol=1e-12))


def pin_shift_invariance(impl):
    """LN(x + c) = LN(x) and the gradients do not change (up to rounding)."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 33))
    dy = rng.standard_normal((4, 33))
    g = rng.uniform(0.5, 1.5, 33)
    b = rng.uniform(-0.5, 0.5, 33)
    y0, _, r0 = impl.forward(x, g, b, EPS)
    y1, _, r1 = impl.forward(x + 7.25, g, b, EPS)
    dx0, dx1 = impl.dx(dy, x, g, EPS), impl.dx(dy, x + 7.25, g, EPS)
    p0, p1 = impl.params(dy, x, EPS), impl.params(dy, x + 7.25, EPS)
    return bool(np.allclose(y0, y1, rtol=0, atol=1e-12) and np.allclose(r0, r1, rtol=1e-12)
                and np.allclose(dx0, dx1, rtol=0, atol=1e-11)
                and all(np.allclose(a, c, rtol=0, atol=1e-11) for a, c in zip(p0, p1)))


def pin_standardised_rows(impl):
    """With gamma = 1 and beta = 0 each output row has mean 0 and mean square
    var / (var + eps)."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((5, 64)) * 3.0 + 1.5
    y, _, _ = impl.forward(x, np.ones(64), None, EPS)
    var = x.var(1)
    return bool(np.allclose(y.mean(1), 0.0, atol=1e-14)
                and np.allclose((y * y).mean(1), var / (var + EPS), rtol=1e-13))


def pin_dx_sums_to_zero(impl):
    """Shift invariance makes every row of dx sum to zero."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal((6, 50))
    dy = rng.standard_normal((6, 50))
    g = rng.uniform(0.5, 1.5, 50)
    return bool(np.allclose(impl.dx(dy, x, g, EPS).sum(1), 0.0, atol=1e-12))


def pin_dbeta_is_column_sum(impl):
    """dbeta is the column sum of dy (not a mean): 17 identical rows give 17
    times one row's value; dgamma scales the same way."""
    rng = np.random.default_rng(11)
    x1 = rng.standard_normal((1, 9))
    dy1 = rng.standard_normal((1, 9))
    g1, b1 = impl.params(dy1, x1, EPS)
    g17, b17 = impl.params(np.repeat(dy1, 17, 0), np.repeat(x1, 17, 0), EPS)
    return bool(np.allclose(b17, 17 * b1, rtol=1e-14) and np.allclose(g17, 17 * g1, rtol=1e-13)
                and np.allclose(b1, dy1[0], rtol=0, atol=0))


def _loss(impl, x, g, b, dy):
    y, _, _ = impl.forward(x, g, b, EPS)
    return float(np.sum(dy * y))


def pin_central_differences(impl):
    """dx, dgamma and dbeta equal the central-difference slopes of
    L = sum(dy * y)."""
    rng = np.random.default_rng(13)
    m, n, h = 3, 7, 1e-6
    x = rng.standard_normal((m, n)) + 0.5
    dy = rng.standard_normal((m, n))
    g = rng.uniform(0.5, 1.5, n)
    b = rng.uniform(-0.5, 0.5, n)
    num_dx = np.zeros_like(x)
    for i in range(m):
        for j in range(n):
            xp, xm = x.copy(), x.copy()
            xp[i, j] += h
            xm[i, j] -= h
            num_dx[i, j] = (_loss(impl, xp, g, b, dy) - _loss(impl, xm, g, b, dy)) / (2 * h)
    num_dg, num_db = np.zeros(n), np.zeros(n)
    for j in range(n):
        gp, gm, bp, bm = g.copy(), g.copy(), b.copy(), b.copy()
        gp[j] += h
        gm[j] -= h
        bp[j] += h
        bm[j] -= h
        num_dg[j] = (_loss(impl, x, gp, b, dy) - _loss(impl, x, gm, b, dy)) / (2 * h)
        num_db[j] = (_loss(impl, x, g, bp, dy) - _loss(impl, x, g, bm, dy)) / (2 * h)
    dg, db = impl.params(dy, x, EPS)
    return bool(np.allclose(impl.dx(dy, x, g, EPS), num_dx, rtol=0, atol=1e-8)
                and np.allclose(dg, num_dg, rtol=0, atol=1e-8)
                and np.allclose(db, num_db, rtol=0, atol=1e-8))


def pin_torch_layer_norm(impl):
    """Agreement with torch.nn.functional.layer_norm and its autograd (fp64)."""
    rng = np.random.default_rng(19)
    for n in (2, 129, 1024):
        x = rng.standard_normal((5, n)) * 2.0 + rng.standard_normal((5, 1))
        dy = rng.standard_normal((5, n))
        g = rng.uniform(0.5, 1.5, n)
        b = rng.uniform(-0.5, 0.5, n)
        xt = torch.tensor(x, requires_grad=True)
        gt = torch.tensor(g, requires_grad=True)
        bt = torch.tensor(b, requires_grad=True)
        yt = torch.nn.functional.layer_norm(xt, (n,), gt, bt, EPS)
        dxt, dgt, dbt = torch.autograd.grad(yt, (xt, gt, bt), torch.tensor(dy))
        y, _, _ = impl.forward(x, g, b, EPS)
        dg, db = impl.params(dy, x, EPS)
        if not np.allclose(y, yt.detach().numpy(), rtol=1e-12, atol=1e-14):
            return False
        if not np.allclose(impl.dx(dy, x, g, EPS), dxt.numpy(), rtol=1e-10, atol=1e-12):
            return False
        if not (np.allclose(dg, dgt.numpy(), rtol=1e-10, atol=1e-12)
                and np.allclose(db, dbt.numpy(), rtol=1e-12, atol=1e-13)):
            return False
    return True


PINS = {
    "two_values": pin_two_values,
    "biased_variance": pin_biased_variance,
    "constant_row": pin_constant_row,
    "shift_invariance": pin_shift_invariance,
    "standardised_rows": pin_standardised_rows,
    "dx_sums_to_zero": pin_dx_sums_to_zero,
    "dbeta_is_column_sum": pin_dbeta_is_column_sum,
    "central_differences": pin_central_differences,
    "torch_layer_norm": pin_torch_layer_norm,
}


@pytest.mark.parametrize("pin", sorted(PINS))
def test_golden_holds_pin(pin):
    assert PINS[pin](GOLDEN), f"golden fails pin {pin}"


CAUGHT_BY = {
    "unbiased_variance": ["two_values", "biased_variance", "standardised_rows",
                          "torch_layer_norm"],
    "not_centred": ["two_values", "shift_invariance", "standardised_rows",
                    "dx_sums_to_zero", "torch_layer_norm"],
    "eps_outside_sqrt": ["constant_row"],
    "beta_dropped": ["two_values", "constant_row", "central_differences", "torch_layer_norm"],
    "dx_without_mean_u": ["constant_row", "dx_sums_to_zero", "central_differences",
                          "torch_layer_norm"],
    "dx_without_xhat_term": ["central_differences", "torch_layer_norm"],
    "dbeta_mean": ["dbeta_is_column_sum"],
    "dgamma_without_r": ["central_differences", "torch_layer_norm"],
}


@pytest.mark.parametrize("mutant,pin", [(m, p) for m, ps in sorted(CAUGHT_BY.items())
                                        for p in ps])
def test_pin_catches_planted_mistake(mutant, pin):
    assert not PINS[pin](MUTANTS[mutant]), f"pin {pin} misses mutant {mutant}"


def test_chunking_and_subsets_agree():
    rng = np.random.default_rng(23)
    x = rng.standard_normal((37, 40)) + 2.0
    dy = rng.standard_normal((37, 40))
    g = rng.uniform(0.5, 1.5, 40)
    b = rng.uniform(-0.5, 0.5, 40)
    y, mu, r = ln.golden_ln_forward(x, g, b, EPS)
    y2, mu2, r2 = ln.golden_ln_forward(x, g, b, EPS, chunk_rows=5)
    rows = [0, 7, 36]
    y3, mu3, r3 = ln.golden_ln_forward(x, g, b, EPS, rows=rows)
    assert np.array_equal(y, y2) and np.array_equal(mu, mu2) and np.array_equal(r, r2)
    assert np.array_equal(y3, y[rows]) and np.array_equal(r3, r[rows])
    dx, dg, db = ln.golden_ln_backward(dy, x, g, EPS)
    assert np.array_equal(ln.golden_ln_dx(dy, x, g, EPS, rows=rows), dx[rows])
    cols = [1, 39]
    dgc, dbc = ln.golden_ln_param_grads(dy, x, EPS, cols=cols, chunk_rows=6)
    assert np.allclose(dgc, dg[cols], rtol=1e-14) and np.allclose(dbc, db[cols], rtol=1e-14)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_reference_is_close_to_golden(dtype):
    """The float32-intermediate reference lands within a few units of its
    output precision of the golden, and its float32 statistics and parameter
    gradients within float32 rounding of a few hundred terms."""
    g_ = torch.Generator().manual_seed(29)
    x = (torch.randn(64, 300, generator=g_) + torch.randn(64, 1, generator=g_)).to(dtype)
    dy = torch.randn(64, 300, generator=g_).to(dtype)
    g = (torch.rand(300, generator=g_) + 0.5).to(dtype)
    b = (torch.rand(300, generator=g_) - 0.5).to(dtype)
    y, mu, r = ln.reference_ln_forward(x, g, b, EPS)
    yg, mug, rg = ln.golden_ln_forward(x, g, b, EPS)
    ulp = {torch.float32: 2.0 ** -23, torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}[dtype]
    assert np.max(np.abs(y.double().numpy() - yg)) <= 4 * ulp * np.max(np.abs(yg))
    assert np.allclose(mu.double().numpy(), mug, rtol=1e-5, atol=1e-6)
    assert np.allclose(r.double().numpy(), rg, rtol=1e-5)
    dx, dgr, dbr = ln.reference_ln_backward(dy, x, g, EPS)
    dxg, dgg, dbg = ln.golden_ln_backward(dy, x, g, EPS)
    assert np.max(np.abs(dx.double().numpy() - dxg)) <= 8 * ulp * np.max(np.abs(dxg))
    assert np.allclose(dgr.double().numpy(), dgg, rtol=1e-4, atol=1e-4)
    assert np.allclose(dbr.double().numpy(), dbg, rtol=1e-5, atol=1e-5)
    dgc, dbc = ln.reference_ln_param_grads(dy, x, EPS, cols=[0, 299])
    assert np.allclose(dgc.numpy(), dgr[[0, 299]].numpy(), rtol=1e-5, atol=1e-4)
    assert np.allclose(dbc.numpy(), dbr[[0, 299]].numpy(), rtol=1e-5, atol=1e-4)


def test_bad_eps_and_shapes_rejected():
    with pytest.raises(ValueError):
        ln.golden_ln_forward(np.ones((2, 3)), np.ones(3), None, 0.0)
    with pytest.raises(ValueError):
        ln.golden_ln_forward(np.ones((2, 3)), np.ones(4))
    with pytest.raises(ValueError):
        ln.golden_ln_dx(np.ones((2, 4)), np.ones((2, 3)), np.ones(3))
