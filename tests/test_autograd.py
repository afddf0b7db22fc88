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
    assert (calls["forward"], calls["backward"]) == (steps, steps)
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


# ---- the other paths: LayerNorm, the fused residual add, the output cast ----

def test_other_functions_reject_cpu_tensors():
    x = torch.randn(4, 64, requires_grad=True)
    w = torch.ones(64, requires_grad=True)
    for call in (lambda: rag.layernorm(x, w), lambda: rag.add_rmsnorm(x, x.detach(), w),
                 lambda: rag.rmsnorm_cast(x, w)):
        with pytest.raises(ValueError):
            call()


def test_other_modules_initial_weights():
    ln = rag.LayerNorm(8)
    assert torch.equal(ln.weight.detach(), torch.ones(8))
    assert torch.equal(ln.bias.detach(), torch.zeros(8))
    assert rag.LayerNorm(8, bias=False).bias is None
    assert torch.equal(rag.AddRMSNorm(8, offset=True).weight.detach(), torch.zeros(8))
    m = rag.RMSNormCast(8, out_dtype=torch.float16)
    assert m.weight.dtype == torch.float32 and m.out_dtype == torch.float16


@pytest.mark.gpu
@pytest.mark.parametrize("bias", [True, False])
def test_layernorm_function_equals_abi_calls(cuda, bias):
    inp = workloads.make_layernorm_inputs("c2", M=129, N=4096)
    x = inp["x"].to(cuda).reshape(3, 43, 4096).requires_grad_(True)
    w = inp["w"].to(cuda).requires_grad_(True)
    b = inp["b"].to(cuda).requires_grad_(True) if bias else None
    dy = inp["dy"].to(cuda).reshape(3, 43, 4096)
    n0 = dict(rag.CALLS)
    y = rag.layernorm(x, w, b, 1e-5)
    y.backward(dy)
    x0, w0 = inp["x"].to(cuda), inp["w"].to(cuda)
    y0, m0, r0 = rn.ln_fwd(x0, w0, inp["b"].to(cuda) if bias else None, 1e-5)
    dx0, dg0, db0 = rn.ln_bwd(dy.reshape(129, 4096), x0, w0, m0, r0, dgamma_dtype=w0.dtype,
                              bias=bias)
    torch.cuda.synchronize()
    assert torch.equal(y.detach().reshape(129, 4096), y0)
    assert torch.equal(x.grad.reshape(129, 4096), dx0)
    assert torch.equal(w.grad, dg0)
    if bias:
        assert torch.equal(b.grad, db0)
    assert rag.CALLS["ln_forward"] == n0["ln_forward"] + 1
    assert rag.CALLS["ln_backward"] == n0["ln_backward"] + 1
    ref = torch.nn.functional.layer_norm(x.detach().float(), (4096,), w.detach().float(),
                                         b.detach().float() if bias else None, 1e-5)
    assert torch.allclose(y.detach().float(), ref, rtol=2 ** -7, atol=2 ** -7)


@pytest.mark.gpu
@pytest.mark.parametrize("use_h", [True, False])
def test_add_rmsnorm_function_equals_abi_calls(cuda, use_h):
    """Both outputs differentiable: x and res receive dRMSNorm/dh (dy) + dh
    (dh absent when h is not used downstream)."""
    inp = workloads.make_add_inputs("c2", M=129, N=4096)
    x = inp["x"].to(cuda).requires_grad_(True)
    res = inp["res"].to(cuda).requires_grad_(True)
    w = inp["w"].to(cuda).requires_grad_(True)
    dy, dh = inp["dy"].to(cuda), inp["dh"].to(cuda)
    y, h = rag.add_rmsnorm(x, res, w)
    if use_h:
        torch.autograd.backward([y, h], [dy, dh])
    else:
        y.backward(dy)
    y0, h0, r0 = rn.add_fwd(inp["x"].to(cuda), inp["res"].to(cuda), inp["w"].to(cuda))
    dx0, dg0 = rn.add_bwd(dy, dh if use_h else None, h0, inp["w"].to(cuda), r0,
                          dgamma_dtype=w.dtype)
    torch.cuda.synchronize()
    assert torch.equal(y.detach(), y0) and torch.equal(h.detach(), h0)
    assert torch.equal(x.grad, dx0) and torch.equal(res.grad, dx0)
    assert x.grad.data_ptr() != res.grad.data_ptr()
    assert torch.equal(w.grad, dg0)


@pytest.mark.gpu
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float16])
def test_rmsnorm_cast_function_equals_abi_calls(cuda, out_dtype):
    inp = workloads.make_cast_inputs("c5", M=129, N=5120, out_dtype=out_dtype)
    x = inp["x"].to(cuda).requires_grad_(True)
    w = inp["w"].to(cuda).requires_grad_(True)
    dy = inp["dy"].to(cuda)
    y = rag.rmsnorm_cast(x, w, out_dtype, 1e-6, True)
    y.backward(dy)
    y0, r0 = rn.cast_fwd(inp["x"].to(cuda), inp["w"].to(cuda), out_dtype, 1e-6, True)
    dx0, dg0 = rn.cast_bwd(dy, inp["x"].to(cuda), inp["w"].to(cuda), r0, True)
    torch.cuda.synchronize()
    assert y.dtype == out_dtype and torch.equal(y.detach(), y0)
    assert x.grad.dtype == torch.float32 and torch.equal(x.grad, dx0)
    assert torch.equal(w.grad, dg0)


@pytest.mark.gpu
def test_layernorm_module_trains_like_torch(cuda):
    """Linear -> LayerNorm -> SiLU -> Linear, 30 Adam steps in float32 beside
    the same network with PyTorch's own LayerNorm, from the same initial
    weights: the losses agree to 1e-3 at every step, and fall."""
    torch.manual_seed(0)

    def net(norm):
        return torch.nn.Sequential(torch.nn.Linear(64, 256), norm, torch.nn.SiLU(),
                                   torch.nn.Linear(256, 8)).to(cuda)

    kern = net(rag.LayerNorm(256, device=cuda))
    ref = net(torch.nn.LayerNorm(256, device=cuda))
    ref.load_state_dict(kern.state_dict())
    opt_k = torch.optim.Adam(kern.parameters(), lr=3e-3)
    opt_r = torch.optim.Adam(ref.parameters(), lr=3e-3)
    g = torch.Generator(device=cuda).manual_seed(1)
    wt = torch.randn(64, 8, device=cuda, generator=g)
    first = None
    for step in range(30):
        xb = torch.randn(32, 64, device=cuda, generator=g)
        yb = torch.tanh(xb @ wt)
        lk = torch.nn.functional.mse_loss(kern(xb), yb)
        lr_ = torch.nn.functional.mse_loss(ref(xb), yb)
        for opt, loss in ((opt_k, lk), (opt_r, lr_)):
            opt.zero_grad()
            loss.backward()
            opt.step()
        first = lk.item() if first is None else first
        assert abs(lk.item() - lr_.item()) <= 1e-3 * max(1.0, lr_.item()), step
    assert lk.item() < 0.5 * first
