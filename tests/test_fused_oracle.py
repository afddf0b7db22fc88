"""Pins of the fused residual-add RMSNorm oracle (oracle.fused): h is the
dtype's own add, the composition reduces to plain RMSNorm, and the backward
(RMSNorm's gradient at h plus the residual stream's dh) equals central
differences and PyTorch's float64 autograd of the unfused composition.
Four planted mistakes (dh dropped or subtracted, the norm of x instead of
h, dgamma without r) are each rejected by the pins named for them."""
import numpy as np
import pytest
import torch

from oracle import fused, golden

EPS = 1e-6


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_residual_sum_is_the_dtype_add(dtype):
    """h equals the exact sum rounded to the dtype, except where the float32
    sum itself rounded first (a double rounding, at most one unit of the
    dtype away); and it is PyTorch's own add."""
    g = torch.Generator().manual_seed(3)
    x = (torch.randn(64, 300, generator=g) * 4).to(dtype)
    r = (torch.randn(64, 300, generator=g) * 4).to(dtype)
    h = fused.residual_sum(x, r)
    assert h.dtype == dtype and torch.equal(h, x + r)
    exact = x.double() + r.double()
    single = exact.to(dtype)
    ulp = {torch.float32: 2.0 ** -23, torch.bfloat16: 2.0 ** -7, torch.float16: 2.0 ** -10}[dtype]
    diff = (h.double() - single.double()).abs()
    assert bool((diff <= ulp * exact.abs().clamp_min(1e-30)).all())
    assert (h == single).float().mean() > 0.99


def test_zero_residual_is_plain_rmsnorm():
    rng = np.random.default_rng(5)
    x = torch.tensor(rng.standard_normal((7, 33)))
    w = torch.tensor(rng.uniform(0.5, 1.5, 33))
    h, y, r = fused.golden_add_forward(x, torch.zeros_like(x), w, EPS)
    y0, r0 = golden.golden_forward(x, w, EPS)
    assert torch.equal(h, x) and np.array_equal(y, y0) and np.array_equal(r, r0)
    dy = torch.tensor(rng.standard_normal((7, 33)))
    dx, dg = fused.golden_add_backward(dy, None, h, w, EPS)
    assert np.array_equal(dx, golden.golden_dx(dy, x, w, EPS))
    assert np.array_equal(dg, golden.golden_dgamma(dy, x, EPS))


def _loss(x, res, w, dy, dh, offset):
    h = x + res
    y, _ = golden.golden_forward(h, w, EPS, offset)
    return float(np.sum(dy * y) + np.sum(dh * h))


class _Oracle:
    """The fused-add oracle under test: forward -> (h, y, r), dx, backward."""
    forward = staticmethod(fused.golden_add_forward)
    dx = staticmethod(fused.golden_add_dx)
    backward = staticmethod(fused.golden_add_backward)


def _central_differences_hold(oracle, offset):
    """dx = d/dx and d/dresidual of L = sum(dy*y) + sum(dh*h), in float64
    (where the add does not round)."""
    rng = np.random.default_rng(7)
    m, n, step = 3, 6, 1e-6
    x, res = rng.standard_normal((m, n)), rng.standard_normal((m, n))
    dy, dh = rng.standard_normal((m, n)), rng.standard_normal((m, n))
    w = rng.standard_normal(n) * 0.02 if offset else rng.uniform(0.5, 1.5, n)
    h, _, _ = oracle.forward(torch.tensor(x), torch.tensor(res), w, EPS, offset)
    dx = oracle.dx(dy, dh, h, w, EPS, offset)
    for target in ("x", "res"):
        num = np.zeros((m, n))
        for i in range(m):
            for j in range(n):
                p, q = (x.copy(), x.copy()) if target == "x" else (res.copy(), res.copy())
                p[i, j] += step
                q[i, j] -= step
                args_p = (p, res) if target == "x" else (x, p)
                args_q = (q, res) if target == "x" else (x, q)
                num[i, j] = (_loss(*args_p, w, dy, dh, offset)
                             - _loss(*args_q, w, dy, dh, offset)) / (2 * step)
        if not np.allclose(dx, num, rtol=0, atol=1e-8):
            return False
    return True


def _autograd_agrees(oracle):
    """y, dx (for x and for the residual) and dgamma against PyTorch's
    float64 autograd of the unfused composition (add, then rms_norm)."""
    rng = np.random.default_rng(11)
    x = torch.tensor(rng.standard_normal((5, 129)), requires_grad=True)
    res = torch.tensor(rng.standard_normal((5, 129)), requires_grad=True)
    w = torch.tensor(rng.uniform(0.5, 1.5, 129), requires_grad=True)
    dy = torch.tensor(rng.standard_normal((5, 129)))
    dh = torch.tensor(rng.standard_normal((5, 129)))
    h = x + res
    y = torch.nn.functional.rms_norm(h, (129,), w, EPS)
    ((y * dy).sum() + (h * dh).sum()).backward()
    hh, yy, _ = oracle.forward(x.detach(), res.detach(), w.detach(), EPS)
    dx, dg = oracle.backward(dy, dh, hh, w.detach(), EPS)
    return (np.allclose(yy, y.detach().numpy(), rtol=1e-13, atol=1e-15)
            and np.allclose(dx, x.grad.numpy(), rtol=1e-11, atol=1e-13)
            and np.allclose(dx, res.grad.numpy(), rtol=1e-11, atol=1e-13)
            and np.allclose(dg, w.grad.numpy(), rtol=1e-11, atol=1e-13))


@pytest.mark.parametrize("offset", [False, True])
def test_central_differences(offset):
    assert _central_differences_hold(_Oracle, offset)


def test_torch_autograd_of_the_unfused_composition():
    assert _autograd_agrees(_Oracle)


# Planted mistakes, each a plausible slip in writing the fused oracle; the
# pins named for it must reject it.
def _h_of(x, res):
    return np.asarray(torch.as_tensor(x).double() + torch.as_tensor(res).double())


class _DroppedDh(_Oracle):  # the residual stream's gradient left out of dx
    @staticmethod
    def dx(dy, dh, h, w, eps, offset=False):
        return golden.golden_dx(dy, h, w, eps, offset)

    @staticmethod
    def backward(dy, dh, h, w, eps, offset=False):
        return golden.golden_dx(dy, h, w, eps, offset), golden.golden_dgamma(dy, h, eps)


class _DhSign(_Oracle):  # dh subtracted instead of added
    @staticmethod
    def dx(dy, dh, h, w, eps, offset=False):
        return golden.golden_dx(dy, h, w, eps, offset) - np.asarray(dh, dtype=np.float64)

    @staticmethod
    def backward(dy, dh, h, w, eps, offset=False):
        return (golden.golden_dx(dy, h, w, eps, offset) - np.asarray(dh, dtype=np.float64),
                golden.golden_dgamma(dy, h, eps))


class _NormOfX(_Oracle):  # the norm taken of x instead of h = x + res
    @staticmethod
    def forward(x, res, w, eps, offset=False):
        y, r = golden.golden_forward(x, w, eps, offset)
        return torch.as_tensor(_h_of(x, res)), y, r


class _DgammaWithoutR(_Oracle):  # dgamma summed as dy*h, the factor r left out
    @staticmethod
    def backward(dy, dh, h, w, eps, offset=False):
        dx = fused.golden_add_dx(dy, dh, h, w, eps, offset)
        hh = np.asarray(torch.as_tensor(h).double())
        return dx, np.sum(np.asarray(torch.as_tensor(dy).double()) * hh, axis=0)


MUTANTS = {"dropped_dh": _DroppedDh, "dh_sign": _DhSign, "norm_of_x": _NormOfX,
           "dgamma_without_r": _DgammaWithoutR}
PINS = {"central_differences": lambda o: _central_differences_hold(o, False),
        "central_differences_offset": lambda o: _central_differences_hold(o, True),
        "autograd": _autograd_agrees}
CAUGHT_BY = {"dropped_dh": ["central_differences", "autograd"],
             "dh_sign": ["central_differences", "central_differences_offset", "autograd"],
             "norm_of_x": ["autograd"],
             "dgamma_without_r": ["autograd"]}


@pytest.mark.parametrize("mutant,pin", [(m, p) for m, ps in sorted(CAUGHT_BY.items())
                                        for p in ps])
def test_pin_catches_planted_mistake(mutant, pin):
    assert not PINS[pin](MUTANTS[mutant]), f"pin {pin} misses mutant {mutant}"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
def test_reference_close_to_golden(dtype):
    g = torch.Generator().manual_seed(13)
    x = torch.randn(32, 500, generator=g).to(dtype)
    res = torch.randn(32, 500, generator=g).to(dtype)
    w = (torch.rand(500, generator=g) + 0.5).to(dtype)
    dy = torch.randn(32, 500, generator=g).to(dtype)
    dh = torch.randn(32, 500, generator=g).to(dtype)
    h, y, r = fused.reference_add_forward(x, res, w, EPS)
    hg, yg, rg = fused.golden_add_forward(x, res, w, EPS)
    assert torch.equal(h, hg)
    ulp = {torch.float32: 2.0 ** -23, torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}[dtype]
    assert np.max(np.abs(y.double().numpy() - yg)) <= 4 * ulp * np.max(np.abs(yg))
    dx, dgr = fused.reference_add_backward(dy, dh, h, w, EPS)
    dxg, dgg = fused.golden_add_backward(dy, dh, h, w, EPS)
    assert np.max(np.abs(dx.double().numpy() - dxg)) <= 4 * ulp * np.max(np.abs(dxg))
    assert np.allclose(dgr.double().numpy(), dgg, rtol=1e-4, atol=1e-4)
