"""Pins of the cast-after-norm oracle (oracle.fused, the output cast fused
after RMSNorm): the page's worked example rounded by hand, PyTorch's own
``rms_norm`` followed by a cast, the float64 golden rounded once, and
PyTorch's float64 autograd through the cast.  Planted mistakes (a
truncating cast, a cast before gamma, a mis-scaled dy) are rejected by the
pins named for them."""
import numpy as np
import pytest
import torch

from oracle import fused, golden

EPS = 1e-6
ULP = {torch.bfloat16: 2.0 ** -7, torch.float16: 2.0 ** -10}
SUBNORMAL_STEP = {torch.bfloat16: 2.0 ** -133, torch.float16: 2.0 ** -24}


# The page "Check an AI model calculation before accelerating it" (section
# "A worked numerical example") prints y = [0.848528, 1.131371] for x = [3, 4],
# gamma = [1, 1], and y = [1.697056, 0.565685] for gamma = [2, 0.5].  Rounded
# to nearest on each dtype's grid (bf16: spacing 2^-8 on [0.5, 1) and 2^-7 on
# [1, 2); fp16: 2^-11 and 2^-10):
#   0.848528 / 2^-8  = 217.22 -> 217 * 2^-8  = 0.84765625
#   1.131371 / 2^-7  = 144.82 -> 145 * 2^-7  = 1.1328125
#   1.697056 / 2^-7  = 217.22 -> 217 * 2^-7  = 1.6953125
#   0.565685 / 2^-8  = 144.82 -> 145 * 2^-8  = 0.56640625
#   0.848528 / 2^-11 = 1737.8 -> 1738 * 2^-11 = 0.8486328125
#   1.131371 / 2^-10 = 1158.5 -> 1159 * 2^-10 = 1.1318359375
#   1.697056 / 2^-10 = 1737.8 -> 1738 * 2^-10 = 1.697265625
#   0.565685 / 2^-11 = 1158.5 -> 1159 * 2^-11 = 0.56591796875
WORKED = {
    (torch.bfloat16, (1.0, 1.0)): [0.84765625, 1.1328125],
    (torch.bfloat16, (2.0, 0.5)): [1.6953125, 0.56640625],
    (torch.float16, (1.0, 1.0)): [0.8486328125, 1.1318359375],
    (torch.float16, (2.0, 0.5)): [1.697265625, 0.56591796875],
}


def _worked_example_holds(forward, key):
    out_dtype, gamma = key
    x = torch.tensor([[3.0, 4.0]])
    y, r = forward(x, torch.tensor(gamma), out_dtype, EPS)
    return (y.dtype == out_dtype and y.double().flatten().tolist() == WORKED[key]
            and abs(float(r[0]) - 0.2828427011609112) < 1e-7)


@pytest.mark.parametrize("key", list(WORKED))
def test_worked_example_rounded(key):
    assert _worked_example_holds(fused.reference_cast_forward, key)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("offset", [False, True])
def test_matches_library_rms_norm_then_cast(out_dtype, offset):
    """PyTorch's ``rms_norm`` in float32, then ``.to``: the same values up to
    one unit of the narrow dtype where the two float32 evaluations straddle a
    rounding boundary (rare)."""
    g = torch.Generator().manual_seed(11)
    x = torch.randn(96, 320, generator=g)
    w = torch.randn(320, generator=g) * 0.02 if offset else torch.rand(320, generator=g) + 0.5
    y, _ = fused.reference_cast_forward(x, w, out_dtype, EPS, offset)
    lib = torch.nn.functional.rms_norm(x, (320,), (1.0 + w) if offset else w, EPS).to(out_dtype)
    d = (y.double() - lib.double()).abs()
    assert bool((d <= ULP[out_dtype] * lib.double().abs()).all())
    assert (y == lib).double().mean() > 0.99


def _golden_rounded_once_holds(forward, out_dtype):
    rng = np.random.default_rng(13)
    x = torch.tensor(rng.standard_normal((64, 257)), dtype=torch.float32)
    w = torch.tensor(rng.uniform(0.5, 1.5, 257), dtype=torch.float32)
    y, _ = forward(x, w, out_dtype, EPS)
    yg, _ = fused.golden_cast_forward(x, w, EPS)
    yg_t = torch.tensor(yg)
    bound = ULP[out_dtype] * yg_t.abs() + SUBNORMAL_STEP[out_dtype]
    return (bool(((y.double() - yg_t).abs() <= bound).all())
            and (y == yg_t.to(out_dtype)).double().mean() > 0.99)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float16])
def test_is_the_golden_rounded_once(out_dtype):
    """Against the float64 golden: within one unit of the narrow dtype (an
    absolute step below its normal range), and equal to the golden's own
    round-to-nearest cast almost everywhere (a truncating cast would differ
    on about half the elements: see the planted mistake below)."""
    assert _golden_rounded_once_holds(fused.reference_cast_forward, out_dtype)


def _truncating_forward(x, w, out_dtype, eps, offset=False):
    """A planted mistake: the same float32 norm, cast toward zero instead of
    to nearest."""
    xf = x.float()
    g = (1.0 + w.float()) if offset else w.float()
    r = torch.rsqrt(xf.square().mean(-1, keepdim=True) + eps)
    y32 = (xf * r * g).numpy()
    nd = np.float16 if out_dtype == torch.float16 else None
    if nd is not None:
        y = y32.astype(nd)
        over = np.abs(y.astype(np.float32)) > np.abs(y32)
        y[over] = np.nextafter(y[over], np.float16(0))
        return torch.from_numpy(y), r.squeeze(-1)
    bits = torch.from_numpy(y32).view(torch.int32) & ~0xFFFF
    return bits.view(torch.float32).to(torch.bfloat16), r.squeeze(-1)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float16])
def test_pins_reject_a_truncating_cast(out_dtype):
    assert not _golden_rounded_once_holds(_truncating_forward, out_dtype)
    keys = [k for k in WORKED if k[0] == out_dtype]
    assert not all(_worked_example_holds(_truncating_forward, k) for k in keys)


def _autograd_through_cast_holds(backward, out_dtype, offset):
    g = torch.Generator().manual_seed(17)
    m, n = 9, 40
    x = torch.randn(m, n, generator=g, dtype=torch.float64)
    w = (torch.randn(n, generator=g, dtype=torch.float64) * 0.02 if offset
         else torch.rand(n, generator=g, dtype=torch.float64) + 0.5)
    dy = torch.randn(m, n, generator=g).to(out_dtype)
    xa = x.clone().requires_grad_(True)
    wa = w.clone().requires_grad_(True)
    y = torch.nn.functional.rms_norm(xa, (n,), (1.0 + wa) if offset else wa, EPS).to(out_dtype)
    y.backward(dy)
    dx, dgamma = backward(dy, x, w, EPS, offset)
    return (np.allclose(dx, xa.grad.numpy(), rtol=1e-12, atol=1e-12)
            and np.allclose(dgamma, wa.grad.numpy(), rtol=1e-12, atol=1e-12))


def _cast_before_gamma_forward(x, w, out_dtype, eps, offset=False):
    """A planted mistake: x*r rounded to the narrow dtype before gamma."""
    xf = x.float()
    g = (1.0 + w.float()) if offset else w.float()
    r = torch.rsqrt(xf.square().mean(-1, keepdim=True) + eps)
    return ((xf * r).to(out_dtype).float() * g).to(out_dtype), r.squeeze(-1)


def _misscaled_dy_backward(dy, x, w, eps, offset=False):
    """A planted mistake: dy taken at twice its value when widened."""
    return fused.golden_cast_backward(dy.double() * 2.0, x, w, eps, offset)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float16])
def test_pins_reject_a_cast_before_gamma_and_a_misscaled_dy(out_dtype):
    assert not _golden_rounded_once_holds(_cast_before_gamma_forward, out_dtype)
    assert not _autograd_through_cast_holds(_misscaled_dy_backward, out_dtype, False)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("offset", [False, True])
def test_backward_is_float64_autograd_through_the_cast(out_dtype, offset):
    """The gradient of y.to(T_out) reaches x as dy widened: PyTorch's float64
    autograd of rms_norm followed by the cast, fed dy in T_out, gives the
    golden dx and dgamma."""
    assert _autograd_through_cast_holds(fused.golden_cast_backward, out_dtype, offset)
    g = torch.Generator().manual_seed(17)
    m, n = 9, 40
    x = torch.randn(m, n, generator=g, dtype=torch.float64)
    w = (torch.randn(n, generator=g, dtype=torch.float64) * 0.02 if offset
         else torch.rand(n, generator=g, dtype=torch.float64) + 0.5)
    dy = torch.randn(m, n, generator=g).to(out_dtype)
    xa = x.clone().requires_grad_(True)
    wa = w.clone().requires_grad_(True)
    y = torch.nn.functional.rms_norm(xa, (n,), (1.0 + wa) if offset else wa, EPS).to(out_dtype)
    y.backward(dy)
    dx, dgamma = fused.golden_cast_backward(dy, x, w, EPS, offset)
    np.testing.assert_allclose(dx, xa.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dgamma, wa.grad.numpy(), rtol=1e-12, atol=1e-12)
    dxr, dgr = fused.reference_cast_backward(dy, x.float(), w.float(), EPS, offset)
    assert dxr.dtype == torch.float32 and dgr.dtype == torch.float32
    np.testing.assert_allclose(dxr.double().numpy(), dx, rtol=1e-4, atol=1e-5)
