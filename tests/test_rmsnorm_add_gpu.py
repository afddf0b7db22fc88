"""RMSNorm with the residual add fused before it, on the GPU through the C
ABI (include/rmsnorm_add.h), against the fused oracle (oracle.fused): h
bitwise equal to the dtype's add, y, rstd, dx (RMSNorm's gradient plus dh)
and dgamma through the gate, at reduced sizes of each recipe, tile and edge
shapes, rows longer than the row-resident limit (full-width rows of up to
128 KiB on the long-row kernels, other layouts on the split-row plan),
misaligned and strided layouts, without dh, and c2, c3, c4, c5 at full size
on every element (c3-c5 also on sampled rows and columns)."""
import pytest
import torch

import backward_rmsnorm_fwd_amd as rn
from backward_rmsnorm_fwd_amd import workloads
from parity import (assert_pass, gate_add_full, gate_add_full_chunked, gate_add_sampled, log,
                    run_add_target, sample_cols, sample_rows)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,M,N", [("c1a", None, None), ("c1c", None, None),
                                      ("c2", 2051, 4096), ("c2", 517, 4104),
                                      ("c3", 3001, 1000), ("c3", 20011, 1024),
                                      ("c5", 1031, 5120), ("c5", 301, 5112),
                                      ("c4", 37, 16384), ("c4", 9, 16376),
                                      ("c4", 9, 65536), ("c5", 33, 20480),
                                      ("c2", 700, 16400)])
def test_recipes(cuda, name, M, N):
    inp = workloads.make_add_inputs(name, M=M, N=N)
    log(f"case add {name} M={inp['M']} N={inp['N']}")
    assert_pass(gate_add_full(inp, run_add_target(inp, cuda)), f"add {name} @ {M}x{N}")


@pytest.mark.parametrize("dtype,N", [(torch.float32, 1), (torch.bfloat16, 2),
                                     (torch.float16, 255), (torch.bfloat16, 257),
                                     (torch.float32, 4095), (torch.bfloat16, 4097),
                                     (torch.float16, 8193), (torch.float32, 16384),
                                     (torch.bfloat16, 16383), (torch.bfloat16, 16385),
                                     (torch.float16, 16386), (torch.float32, 16388),
                                     (torch.float32, 24577), (torch.bfloat16, 131072)])
def test_edge_shapes(cuda, dtype, N):
    inp = workloads.make_add_inputs("c1a", M=7, N=N, dtype=dtype)
    log(f"case add edge {dtype} N={N}")
    assert_pass(gate_add_full(inp, run_add_target(inp, cuda)), f"add edge {dtype} N={N}")


@pytest.mark.parametrize("N", [4096, 40000])
def test_without_dh(cuda, N):
    inp = workloads.make_add_inputs("c2", M=700 if N == 4096 else 40, N=N)
    out = run_add_target(inp, cuda, with_dh=False)
    assert_pass(gate_add_full(inp, out, with_dh=False), f"add without dh N={N}")


def test_full_size_c2(cuda):
    inp = workloads.make_add_inputs("c2")
    log("case add c2 full size generated")
    out = run_add_target(inp, cuda)
    log("case add c2 device run done")
    assert_pass(gate_add_full(inp, out), "add c2 full size, every element")


@pytest.mark.parametrize("name,nrows", [("c3", 1024), ("c4", 256), ("c5", 1024)])
def test_full_size_sampled(cuda, name, nrows):
    """The fp16 262144 x 1024, bf16 2048 x 65536 (split rows) and offset
    bf16 65536 x 5120 shapes at full size, default plan; sampled rows and
    dgamma columns against the oracle."""
    inp = workloads.make_add_inputs(name)
    log(f"case add {name} full size M={inp['M']} N={inp['N']} generated")
    out = run_add_target(inp, cuda)
    log(f"case add {name} device run done")
    rows = sample_rows(inp, nrows)
    cols = sample_cols(inp["N"], 64)
    assert_pass(gate_add_sampled(inp, out, rows, cols), f"add {name} full size, sampled")
    for k in ("y", "h", "dx", "rstd", "dgamma"):
        assert not torch.isnan(out[k]).any(), f"{k} has unwritten (NaN) elements"


@pytest.mark.parametrize("name", ["c3", "c4", "c5"])
def test_full_size_every_element_chunked(cuda, name):
    """The c3, c4 and c5 shapes at full size in the default plan: h
    bit-exact and every element of y, rstd, dx and dgamma gated, the oracle
    a block of rows at a time."""
    inp = workloads.make_add_inputs(name)
    log(f"case add {name} full size M={inp['M']} N={inp['N']} generated")
    out = run_add_target(inp, cuda)
    log(f"case add {name} device run done")
    assert_pass(gate_add_full_chunked(inp, out), f"add {name} full size, every element")


def test_reproducible_offset_and_dgamma_in_dtype(cuda):
    inp = workloads.make_add_inputs("c5", M=999, N=5120)
    x, res, w, dy, dh = (inp[k].to(cuda) for k in ("x", "res", "w", "dy", "dh"))
    y0, h0, r0 = rn.add_fwd(x, res, w, 1e-6, True)
    runs = [rn.add_bwd(dy, dh, h0, w, r0, True) for _ in range(3)]
    y1, h1, r1 = rn.add_fwd(x, res, w, 1e-6, True)
    assert torch.equal(y0, y1) and torch.equal(h0, h1) and torch.equal(r0, r1)
    for dx, dg in runs[1:]:
        assert torch.equal(dx, runs[0][0]) and torch.equal(dg, runs[0][1])
    dxT, dgT = rn.add_bwd(dy, dh, h0, w, r0, True, dgamma_dtype=x.dtype, poison=True)
    torch.cuda.synchronize()
    assert torch.equal(dxT, runs[0][0]) and torch.equal(dgT, runs[0][1].to(x.dtype))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("M,N", [(33, 4096), (9, 20000)])
def test_misaligned_and_strided(cuda, dtype, M, N):
    inp = workloads.make_add_inputs("c2", M=M, N=N, dtype=dtype)

    def shifted(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=cuda)
        v = buf[1:].view(t.shape)
        v.copy_(t.to(cuda))
        return v

    x, res, w, dy, dh = (shifted(inp[k]) for k in ("x", "res", "w", "dy", "dh"))
    y, h, rstd = rn.add_fwd(x, res, w, inp["eps"], poison=True)
    dx, dg = rn.add_bwd(dy, dh, h, w, rstd, poison=True)
    torch.cuda.synchronize()
    out = {"y": y, "h": h, "rstd": rstd, "dx": dx, "dgamma": dg}
    assert_pass(gate_add_full(inp, out), f"add misaligned {dtype}")

    wide = torch.full((M, 3 * N), -5.0, dtype=dtype, device=cuda)
    wide[:, :N] = inp["x"].to(cuda)
    wide[:, N:2 * N] = inp["res"].to(cuda)
    xs, rs = wide[:, :N], wide[:, N:2 * N]
    hs = wide[:, 2 * N:]  # h written into the third slice of the same buffer
    ys = torch.full((M, N), float("nan"), dtype=dtype, device=cuda)
    r2 = torch.empty(M, device=cuda)
    rn.rmsnorm_add_fwd(xs, rs, inp["w"].to(cuda), inp["eps"], ys, hs, r2)
    dx2, dg2 = rn.add_bwd(inp["dy"].to(cuda), inp["dh"].to(cuda), hs, inp["w"].to(cuda), r2,
                          poison=True)
    torch.cuda.synchronize()
    out2 = {"y": ys, "h": hs.contiguous(), "rstd": r2, "dx": dx2, "dgamma": dg2}
    assert_pass(gate_add_full(inp, out2), f"add strided {dtype}")


def test_m_zero_and_rejections(cuda):
    x = torch.empty((0, 64), device=cuda, dtype=torch.bfloat16)
    w = torch.ones(64, device=cuda, dtype=torch.bfloat16)
    y, h, r = rn.add_fwd(x, x, w)
    dx, dg = rn.add_bwd(x, None, h, w, r, poison=True)
    torch.cuda.synchronize()
    assert torch.equal(dg.cpu(), torch.zeros(64))
    n = rn.RMSNORM_ADD_MAX_N + 1
    t = torch.empty(2, n, device=cuda, dtype=torch.bfloat16)
    with pytest.raises(rn.RmsnormError):
        rn.add_fwd(t, t, torch.ones(n, device=cuda, dtype=torch.bfloat16))
