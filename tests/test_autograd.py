"""The autograd wrapper (backward_rmsnorm_fwd_amd.autograd) and the small
network integration of the page "Check an AI model calculation before
accelerating it", section "Connecting Autograd and actually training":
Linear -> RMSNorm -> SiLU -> Linear trained 100 Adam steps on 32 synthetic
examples per step, beside a reference network with the same initial weights
whose RMSNorm is the eager float32 formula; then the weights are reloaded and
the call counters checked.
"""
import io

import numpy as np
import pytest
import torch

import backward_rmsnorm_fwd_amd as rn
from backward_rmsnorm_fwd_amd import autograd as rag
from backward_rmsnorm_fwd_amd import workloads
from parity import assert_pass, gate_full, log


def test_cpu_tensors_are_rejected_not_rerouted():
    """No CPU path: the wrapper raises instead of computing elsewhere."""
    x = torch.randn(4, 64, requires_grad=True)
    w = torch.ones(64, requires_grad=True)
    with pytest.raises(ValueError):
        rag.rmsnorm(x, w)


def test_module_initial_weights():
    assert torch.equal(rag.RMSNorm(8).weight.detach(), torch.ones(8))
    m = rag.RMSNorm(8, offset=True)
    assert torch.equal(m.weight.detach(), torch.zeros(8)) and m.offset


@pytest.mark.gpu
@pytest.mark.parametrize("name,M,N", [("c5", 301, 5120), ("c2", 129, 4096), ("c1a", 65, 128)])
def test_function_equals_abi_calls_and_passes_gate(cuda, name, M, N):
    """Through autograd the outputs are exactly those of rmsnorm_fwd /
    rmsnorm_bwd (gated against the oracle), dgamma cast to the weight's
    dtype."""
    inp = workloads.make_inputs(name, M=M, N=N)
    off, eps = inp["offset"], inp["eps"]
    x = inp["x"].to(cuda).requires_grad_(True)
    w = inp["w"].to(cuda).requires_grad_(True)
    dy = inp["dy"].to(cuda)
    y = rag.rmsnorm(x, w, eps, off)
    y.backward(dy)
    y0, r0 = rn.fwd(inp["x"].to(cuda), inp["w"].to(cuda), eps, off)
    dx0, dg0 = rn.bwd(dy, inp["x"].to(cuda), inp["w"].to(cuda), r0, off)
    torch.cuda.synchronize()
    assert torch.equal(y.detach(), y0)
    assert torch.equal(x.grad, dx0)
    assert w.grad.dtype == w.dtype and torch.equal(w.grad, dg0.to(w.dtype))
    log(f"case autograd {name} M={M} N={N}")
    assert_pass(gate_full(inp, {"y": y0, "rstd": r0, "dx": dx0, "dgamma": dg0}), f"autograd {name}")


@pytest.mark.gpu
def test_leading_dims_and_strided_input(cuda):
    """A (B, T, N) input and a non-contiguous view give the same result as
    the contiguous 2-D call."""
    g = torch.Generator().manual_seed(5)
    base = torch.randn(6, 256, 4, generator=g).to(cuda)
    xv = base.transpose(1, 2)  # (6, 4, 256), not contiguous
    w = (torch.rand(256, generator=g) + 0.5).to(cuda)
    xa = xv.detach().clone().requires_grad_(True)
    xb = xv.contiguous().reshape(24, 256).detach().requires_grad_(True)
    dy = torch.randn(6, 4, 256, generator=g).to(cuda)
    ya = rag.rmsnorm(xa, w)
    yb = rag.rmsnorm(xb, w)
    ya.backward(dy)
    yb.backward(dy.reshape(24, 256))
    assert ya.shape == (6, 4, 256)
    assert torch.equal(ya.reshape(24, 256), yb)
    assert torch.equal(xa.grad.reshape(24, 256), xb.grad)


class _EagerRMSNorm(torch.nn.Module):
    """Reference path: the eager float32 formula, differentiated by autograd."""

    def __init__(self, dim, eps):
        super().__init__()
        self.weight = torch.nn.Parameter(torch.ones(dim))
        self.eps = eps

    def forward(self, x):
        r = torch.rsqrt(x.float().square().mean(-1, keepdim=True) + self.eps)
        return (x.float() * r * self.weight.float()).to(x.dtype)


def _network(norm, d_in, d_hidden, d_out):
    return torch.nn.Sequential(torch.nn.Linear(d_in, d_hidden), norm, torch.nn.SiLU(),
                               torch.nn.Linear(d_hidden, d_out))


@pytest.mark.gpu
def test_small_network_trains_with_the_kernels(cuda):
    d_in, d_hidden, d_out, eps = 32, 256, 8, 1e-6
    steps, batch = 100, 32
    rng = np.random.default_rng(7)
    teacher = rng.standard_normal((d_in, d_out)).astype(np.float32) / np.sqrt(d_in)
    x_all = rng.standard_normal((steps * batch + 512, d_in)).astype(np.float32)
    noise = rng.standard_normal((x_all.shape[0], d_out))
    y_all = (np.tanh(x_all @ teacher) + 0.05 * noise).astype(np.float32)
    xs = torch.from_numpy(x_all).to(cuda)
    ys = torch.from_numpy(y_all).to(cuda)
    x_test, y_test = xs[-512:], ys[-512:]

    torch.manual_seed(0)
    kern = _network(rag.RMSNorm(d_hidden, eps), d_in, d_hidden, d_out).to(cuda)
    ref = _network(_EagerRMSNorm(d_hidden, eps), d_in, d_hidden, d_out).to(cuda)
    ref.load_state_dict(kern.state_dict())  # identical starting points

    # Initial agreement of outputs and gradients.
    xb, yb = xs[:batch], ys[:batch]
    out_k, out_r = kern(xb), ref(xb)
    torch.nn.functional.mse_loss(out_k, yb).backward()
    torch.nn.functional.mse_loss(out_r, yb).backward()
    out_err = (out_k - out_r).abs().max().item()
    grad_err = max((pk.grad - pr.grad).abs().max().item()
                   for pk, pr in zip(kern.parameters(), ref.parameters()))
    log(f"initial output error {out_err:.3g}, gradient error {grad_err:.3g}")
    assert out_err < 1e-5 and grad_err < 1e-5
    kern.zero_grad()
    ref.zero_grad()

    def mse(model):
        with torch.no_grad():
            return torch.nn.functional.mse_loss(model(x_test), y_test).item()

    start = mse(kern)
    rag.CALLS.update(forward=0, backward=0)
    opt_k = torch.optim.Adam(kern.parameters(), lr=3e-3)
    opt_r = torch.optim.Adam(ref.parameters(), lr=3e-3)
    for step in range(steps):
        xb, yb = xs[step * batch:(step + 1) * batch], ys[step * batch:(step + 1) * batch]
        for model, opt in ((kern, opt_k), (ref, opt_r)):
            opt.zero_grad()
            torch.nn.functional.mse_loss(model(xb), yb).backward()
            opt.step()
    calls = dict(rag.CALLS)
    end_k, end_r = mse(kern), mse(ref)
    log(f"test MSE: start {start:.5f}, kernel path {end_k:.5f}, reference {end_r:.5f}; "
        f"calls {calls}")
    assert calls == {"forward": steps, "backward": steps}
    assert end_k < 0.5 * start
    assert abs(end_k - end_r) <= 1e-3 * end_r

    # Reload the trained weights into a fresh network: identical predictions.
    buf = io.BytesIO()
    torch.save(kern.state_dict(), buf)
    buf.seek(0)
    again = _network(rag.RMSNorm(d_hidden, eps), d_in, d_hidden, d_out).to(cuda)
    again.load_state_dict(torch.load(buf, weights_only=True))
    with torch.no_grad():
        assert torch.equal(again(x_test), kern(x_test))
