"""Edge cases of the long-row and split-row paths of all four families on
the GPU, gated against their oracles: one and two rows (a single row block,
a forward two-row step with one row), rows just past 16384 and past 65536,
the offset weight, and dgamma (dbeta) in the input dtype, which must equal
the float32 result rounded once."""
import pytest
import torch

import backward_rmsnorm_fwd_amd as rn
from backward_rmsnorm_fwd_amd import workloads
from parity import (assert_pass, gate_add_full, gate_cast_full, gate_full, gate_ln_full, log,
                    run_add_target, run_cast_target, run_ln_target, run_target)

pytestmark = pytest.mark.gpu

SHAPES = [(1, 16385), (2, 16392), (1, 65536), (2, 65537), (3, 40000)]


@pytest.mark.parametrize("M,N", SHAPES)
@pytest.mark.parametrize("offset", [False, True])
def test_rmsnorm_few_long_rows(cuda, M, N, offset):
    inp = workloads.make_tile_case((M, N), torch.bfloat16, 90 + M)
    inp["offset"] = offset
    log(f"case rmsnorm few long rows {M}x{N} offset={offset}")
    out = run_target(inp, cuda)
    assert_pass(gate_full(inp, out), f"rmsnorm {M}x{N} offset={offset}")
    x, w, dy = (inp[k].to(cuda) for k in ("x", "w", "dy"))
    dxT, dgT = rn.bwd(dy, x, w, out["rstd"], offset, dgamma_dtype=x.dtype, poison=True)
    torch.cuda.synchronize()
    assert torch.equal(dxT, out["dx"]) and torch.equal(dgT, out["dgamma"].to(x.dtype))


@pytest.mark.parametrize("M,N", SHAPES)
def test_layernorm_few_long_rows(cuda, M, N):
    inp = workloads.make_layernorm_tile_case((M, N), torch.bfloat16, 91 + M)
    log(f"case layernorm few long rows {M}x{N}")
    out = run_ln_target(inp, cuda)
    assert_pass(gate_ln_full(inp, out), f"layernorm {M}x{N}")
    x, w, dy = (inp[k].to(cuda) for k in ("x", "w", "dy"))
    dxT, dgT, dbT = rn.ln_bwd(dy, x, w, out["mean"], out["rstd"], dgamma_dtype=x.dtype,
                              poison=True)
    torch.cuda.synchronize()
    assert torch.equal(dxT, out["dx"])
    assert torch.equal(dgT, out["dgamma"].to(x.dtype)) and torch.equal(dbT, out["dbeta"].to(x.dtype))


@pytest.mark.parametrize("M,N", SHAPES)
@pytest.mark.parametrize("offset", [False, True])
def test_fused_add_few_long_rows(cuda, M, N, offset):
    inp = workloads.make_add_inputs("c1a", M=M, N=N, dtype=torch.bfloat16)
    inp["offset"] = offset
    log(f"case add few long rows {M}x{N} offset={offset}")
    out = run_add_target(inp, cuda)
    assert_pass(gate_add_full(inp, out), f"add {M}x{N} offset={offset}")
    dy, dh, w = (inp[k].to(cuda) for k in ("dy", "dh", "w"))
    dxT, dgT = rn.add_bwd(dy, dh, out["h"], w, out["rstd"], offset, dgamma_dtype=dy.dtype,
                          poison=True)
    torch.cuda.synchronize()
    assert torch.equal(dxT, out["dx"]) and torch.equal(dgT, out["dgamma"].to(dy.dtype))


@pytest.mark.parametrize("M,N", SHAPES)
def test_cast_few_long_rows(cuda, M, N):
    inp = workloads.make_cast_tile_case((M, N), torch.bfloat16, 92 + M)
    log(f"case cast few long rows {M}x{N}")
    assert_pass(gate_cast_full(inp, run_cast_target(inp, cuda)), f"cast {M}x{N}")
