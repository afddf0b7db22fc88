"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

The gate (oracle.gate) is the torchtitan kernel-numerics-verifier criterion:
target_error <= 2.0 * reference_error + rounding_floor(dtype) per tensor, with
structure and conditioning checks, plus rstd within 1e-6 relative of the
float64 golden.  Outputs are pre-filled with NaN so an unwritten element fails
the structure check.  Shapes: the five workloads (small ones whole, the large
ones at reduced M with ragged tails, and at full size on sampled rows and
columns), the torchtitan page's tile-boundary and adversarial-variance cases
(section "形状选择" and "对抗样本"), and the contract's edge cases.
"""
import numpy as np
import pytest
import torch

import backward_rmsnorm_fwd_amd as rn
from backward_rmsnorm_fwd_amd import workloads
from parity import (assert_pass, gate_full, gate_full_chunked, gate_sampled, log, run_target,
                    sample_cols, sample_rows)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["c1a", "c1b", "c1c"])
def test_small_workloads(cuda, name):
    inp = workloads.make_inputs(name)
    log(f"case {name} M={inp['M']} N={inp['N']}")
    assert_pass(gate_full(inp, run_target(inp, cuda)), name)


def test_worked_example_values(cuda):
    """The page's printed y and dx for x=[3,4] (section "Let's work through
    two values" and "Input backward pass: keep the right N")."""
    b = run_target(workloads.make_inputs("c1b"), cuda)
    c = run_target(workloads.make_inputs("c1c"), cuda)
    assert np.allclose(b["y"].cpu().numpy(), [[0.848528, 1.131371]], atol=6e-7)
    assert np.allclose(c["y"].cpu().numpy(), [[1.697056, 0.565685]], atol=6e-7)
    assert np.allclose(b["dx"].cpu().numpy(), [[-0.090510, 0.067882]], atol=6e-7)


TILE_CASES = [((3, 255), torch.float32, 1), ((3, 256), torch.bfloat16, 2),
              ((3, 257), torch.bfloat16, 3), ((3, 257), torch.float16, 10),
              ((8, 6, 256), torch.bfloat16, 4), ((8, 4095), torch.bfloat16, 5),
              ((8, 4096), torch.bfloat16, 6), ((8, 4097), torch.bfloat16, 7),
              ((8, 5120), torch.bfloat16, 8), ((37, 2048), torch.float32, 12),
              ((13, 1100), torch.float32, 13), ((11, 3000), torch.float16, 14),
              ((7, 8200), torch.bfloat16, 15), ((6, 20000), torch.float32, 16),
              ((5, 40000), torch.float16, 17), ((9, 2560), torch.float32, 18),
              ((9, 5120), torch.float16, 19),
              # Long rows that are whole 8 KiB sweeps (3, 4 and 8 chunks),
              # more rows than workgroups: some take two rows, some one.
              ((300, 12288), torch.bfloat16, 20), ((270, 8192), torch.float32, 21),
              ((513, 32768), torch.float16, 22)]


@pytest.mark.parametrize("shape,dtype,seed", TILE_CASES)
def test_tile_boundary_shapes(cuda, shape, dtype, seed):
    inp = workloads.make_tile_case(shape, dtype, seed)
    log(f"case tile {shape} {dtype} seed {seed}")
    assert_pass(gate_full(inp, run_target(inp, cuda)), f"tile {shape} {dtype}")


@pytest.mark.parametrize("seed,scale", [(9, 1e-5), (11, 0.0)])
def test_adversarial_variance(cuda, seed, scale):
    inp = workloads.make_tile_case((8, 5120), torch.bfloat16, seed, scale=scale)
    log(f"case variance scale={scale}")
    assert_pass(gate_full(inp, run_target(inp, cuda)), f"variance scale {scale}")


# Each recipe at reduced M (several workgroups' row blocks and a ragged last
# block) and, where the recipe's N is a multiple of the vector tile, also at
# an N with a ragged last chunk.
# The pipelined kernels interleave row groups over workgroups; 12293 rows of
# 4096 give workgroups 4 or 3 steps (both loop tails) and a last row group
# with 5 of 8 rows.
SCALED = [("c2", 2051, 4096), ("c2", 12293, 4096), ("c2", 517, 4104), ("c3", 20011, 1024),
          ("c3", 3001, 1000), ("c4", 37, 65536), ("c4", 9, 65528), ("c5", 1031, 5120),
          ("c5", 301, 5112)]


@pytest.mark.parametrize("name,M,N", SCALED)
def test_scaled_workloads(cuda, name, M, N):
    inp = workloads.make_inputs(name, M=M, N=N)
    log(f"case {name} recipe at M={M} N={N}")
    assert_pass(gate_full(inp, run_target(inp, cuda)), f"{name} @ {M}x{N}")


@pytest.mark.parametrize("name", ["c2", "c4"])
def test_full_size_every_element(cuda, name):
    """Full-size workload, default plan (the one bench.py times), all
    134M elements of y and dx and all of rstd and dgamma gated against the
    oracle: errors that only appear with the whole GPU loaded cannot hide."""
    inp = workloads.make_inputs(name)
    log(f"case {name} full size M={inp['M']} N={inp['N']} generated")
    out = run_target(inp, cuda)
    log(f"case {name} device run done")
    assert_pass(gate_full(inp, out), f"{name} full size, every element")


@pytest.mark.parametrize("name", ["c3", "c5"])
def test_full_size_every_element_chunked(cuda, name):
    """fp16 262144 x 1024 (special rows included) and bf16 offset 65536 x
    5120, default plan (the one bench.py times, the pipelined backward with
    its explicit waits): every element of y, rstd, dx and dgamma gated, the
    oracle evaluated one block of rows at a time and the blocks' errors
    combined into one gate row per tensor."""
    inp = workloads.make_inputs(name)
    log(f"case {name} full size M={inp['M']} N={inp['N']} generated")
    out = run_target(inp, cuda)
    log(f"case {name} device run done")
    assert_pass(gate_full_chunked(inp, out), f"{name} full size, every element")


@pytest.mark.parametrize("name", ["c3", "c5"])
def test_full_size_sampled(cuda, name):
    """Full-size workload, default plan; y, rstd, dx gated on 2048 sampled
    rows (plus the recipe's special rows), dgamma on sampled columns summed
    over all rows."""
    inp = workloads.make_inputs(name)
    log(f"case {name} full size M={inp['M']} N={inp['N']} generated")
    out = run_target(inp, cuda)
    log(f"case {name} device run done")
    rows = sample_rows(inp, 2048)
    cols = sample_cols(inp["N"], 64)
    assert_pass(gate_sampled(inp, out, rows, cols), f"{name} full size, sampled")
    for k in ("y", "dx", "rstd", "dgamma"):
        assert not torch.isnan(out[k]).any(), f"{k} has unwritten (NaN) elements"


def test_backward_is_bitwise_reproducible(cuda):
    # c3's shape takes the pipelined backward with dy prefetched into
    # registers; the others the row-block, LDS-staged and long-row kernels.
    for name, M, N in [("c2", 4096, 4096), ("c5", 999, 5120), ("c4", 21, 65536),
                       ("c4", 40, 131072), ("c3", 65536, 1024), ("c3", 9001, 512)]:
        inp = workloads.make_inputs(name, M=M, N=N)
        x, w, dy = (inp[k].to(cuda) for k in ("x", "w", "dy"))
        y0, r0 = rn.fwd(x, w, inp["eps"], inp["offset"])
        runs = [rn.bwd(dy, x, w, r0, inp["offset"]) for _ in range(3)]
        y1, r1 = rn.fwd(x, w, inp["eps"], inp["offset"])
        assert torch.equal(y0, y1) and torch.equal(r0, r1)
        for dx, dg in runs[1:]:
            assert torch.equal(dx, runs[0][0]) and torch.equal(dg, runs[0][1]), name


@pytest.mark.parametrize("M,N", [(1500, 4096), (70, 131072)])
def test_stage_entry_points_match_combined(cuda, M, N):
    inp = workloads.make_inputs("c2", M=M, N=N)
    x, w, dy = (inp[k].to(cuda) for k in ("x", "w", "dy"))
    _, r = rn.fwd(x, w)
    dx, dg = rn.bwd(dy, x, w, r)
    m, n = x.shape
    ws = torch.empty(rn.rmsnorm_bwd_workspace_bytes(m, n, x.dtype) // 4, device=cuda)
    dx2 = torch.empty_like(x)
    dg2 = torch.empty(n, device=cuda)
    rn.rmsnorm_bwd_rows(dy, x, w, r, dx2, ws)
    rn.rmsnorm_bwd_reduce(ws, m, n, x.dtype, dg2)
    torch.cuda.synchronize()
    assert torch.equal(dx, dx2) and torch.equal(dg, dg2)


@pytest.mark.parametrize("name,M,N", [("c2", 1500, 4096), ("c3", 3001, 1000), ("c5", 301, 5120),
                                    ("c4", 9, 65528)])
def test_dgamma_in_input_dtype(cuda, name, M, N):
    """With RMSNORM_FLAG_DGAMMA_IN_DTYPE dgamma is the float32 result rounded
    to nearest even to the input dtype (combined call and stage 2 alone)."""
    inp = workloads.make_inputs(name, M=M, N=N)
    x, w, dy = (inp[k].to(cuda) for k in ("x", "w", "dy"))
    off = inp["offset"]
    _, r = rn.fwd(x, w, inp["eps"], off)
    dx, dg32 = rn.bwd(dy, x, w, r, off)
    dx2, dgT = rn.bwd(dy, x, w, r, off, poison=True, dgamma_dtype=x.dtype)
    ws = torch.empty(rn.rmsnorm_bwd_workspace_bytes(M, N, x.dtype, off) // 4, device=cuda)
    rn.rmsnorm_bwd_rows(dy, x, w, r, torch.empty_like(x), ws, off)
    dgT2 = torch.full((N,), float("nan"), device=cuda, dtype=x.dtype)
    rn.rmsnorm_bwd_reduce(ws, M, N, x.dtype, dgT2, off)
    torch.cuda.synchronize()
    assert dgT.dtype == x.dtype
    assert torch.equal(dx, dx2)
    assert torch.equal(dgT, dg32.to(x.dtype)) and torch.equal(dgT2, dgT)


# (recipe, M, N, row stride of x/dy, row stride of y/dx): full-width kernels
# (16-byte aligned strides), the long-row kernel, and odd strides that force
# narrower vectors.
STRIDED = [("c2", 1500, 4096, 4104, 4160), ("c3", 3001, 1000, 1003, 1024),
           ("c5", 301, 5120, 5200, 5128), ("c4", 9, 65528, 65536, 65600),
           ("c1a", 65, 128, 130, 129), ("c4", 19, 98304, 98305, 98312),
           ("c3", 9, 70000, 70008, 70001)]


@pytest.mark.parametrize("name,M,N,ldi,ldo", STRIDED)
def test_strided_rows(cuda, name, M, N, ldi, ldo):
    """x and dy are column slices of wider buffers, y and dx are written into
    wider buffers; the gaps between rows are never touched."""
    inp = workloads.make_inputs(name, M=M, N=N)
    off, eps = inp["offset"], inp["eps"]
    T = inp["x"].dtype
    sentinel = -12345.0

    def sliced(t, ld):
        buf = torch.full((M, ld), sentinel, dtype=T, device=cuda)
        buf[:, :N] = t.to(cuda)
        return buf, buf[:, :N]

    xbuf, x = sliced(inp["x"], ldi)
    dybuf, dy = sliced(inp["dy"], ldi)
    ybuf = torch.full((M, ldo), float("nan"), dtype=T, device=cuda)
    dxbuf = torch.full((M, ldo), float("nan"), dtype=T, device=cuda)
    ybuf[:, N:] = sentinel
    dxbuf[:, N:] = sentinel
    y, dx = ybuf[:, :N], dxbuf[:, :N]
    w = inp["w"].to(cuda)
    rstd = torch.full((M,), float("nan"), device=cuda)
    dg = torch.full((N,), float("nan"), device=cuda)
    ws = torch.empty(max(4, rn.rmsnorm_bwd_workspace_bytes(M, N, T, off)) // 4, device=cuda)
    log(f"case strided {name} M={M} N={N} ld {ldi}/{ldo}")
    rn.rmsnorm_fwd_strided(x, w, eps, y, rstd, off)
    rn.rmsnorm_bwd_strided(dy, x, w, rstd, dx, dg, ws, off)
    torch.cuda.synchronize()
    for buf in (ybuf, dxbuf):
        assert bool((buf[:, N:] == sentinel).all()), "a gap between rows was written"
    for buf in (xbuf, dybuf):
        assert bool((buf[:, N:] == sentinel).all()), "an input gap was written"
    out = {"y": y.contiguous(), "rstd": rstd, "dx": dx.contiguous(), "dgamma": dg}
    assert_pass(gate_full(inp, out), f"strided {name}")


def test_output_interleaved_with_input(cuda):
    """x in the first N columns of a buffer, y in the next N (same row stride):
    accepted as disjoint and computed correctly."""
    inp = workloads.make_inputs("c2", M=777, N=4096)
    buf = torch.empty((777, 2 * 4096), dtype=torch.bfloat16, device=cuda)
    buf[:, :4096] = inp["x"].to(cuda)
    x, y = buf[:, :4096], buf[:, 4096:]
    rstd = torch.empty(777, device=cuda)
    rn.rmsnorm_fwd_strided(x, inp["w"].to(cuda), inp["eps"], y, rstd)
    y0, r0 = rn.fwd(inp["x"].to(cuda), inp["w"].to(cuda), inp["eps"])
    torch.cuda.synchronize()
    assert torch.equal(y, y0) and torch.equal(rstd, r0)
    assert torch.equal(x, inp["x"].to(cuda))


def test_side_stream(cuda):
    inp = workloads.make_inputs("c3", M=5000, N=1024)
    x, w, dy = (inp[k].to(cuda) for k in ("x", "w", "dy"))
    y0, r0 = rn.fwd(x, w)
    dx0, dg0 = rn.bwd(dy, x, w, r0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        y1, r1 = rn.fwd(x, w, stream=s)
        dx1, dg1 = rn.bwd(dy, x, w, r1, stream=s)
    s.synchronize()
    assert torch.equal(y0, y1) and torch.equal(dx0, dx1) and torch.equal(dg0, dg1)


# Rows longer than 65536 elements take the split-row plan: 16 KiB segments
# (4096 fp32 / 8192 16-bit elements) over several workgroups, stats -> finish
# -> apply.  Cases: a last segment of 1 element with 2-byte accesses (fp16
# N=65537), 17 segments with a 4-element tail (fp32 N=65540), one row per
# block (M=3), odd M (the two-row steps' tail), blocks of 16+ rows, the
# recipes' special rows (c3) and offset weight (c5), and the largest N.
# Stage 2 then runs with 1, 2, 4, 8 and 16 slices of partial rows.
SPLIT_TILES = [((5, 65537), torch.float16, 21), ((7, 65540), torch.float32, 22),
               ((3, 1 << 20), torch.bfloat16, 23), ((2, rn.MAX_N), torch.bfloat16, 24),
               ((4, 3, 100003), torch.float16, 25), ((11, 200000), torch.float32, 26),
               ((30, 327680), torch.bfloat16, 27)]
SPLIT_RECIPES = [("c4", 33, 131072), ("c4", 261, 98304), ("c3", 301, 70000),
                 ("c5", 129, 81920), ("c2", 600, 73728)]


@pytest.mark.parametrize("shape,dtype,seed", SPLIT_TILES)
def test_split_rows_tiles(cuda, shape, dtype, seed):
    plan = rn.rmsnorm_query_plan(int(np.prod(shape[:-1])), shape[-1], dtype,
                                 which=rn.PASS_BWD_ROWS)
    assert plan["kernel_name"] == "bwd_split"
    inp = workloads.make_tile_case(shape, dtype, seed)
    log(f"case split {shape} {dtype} seed {seed} segments {plan['segments']}")
    assert_pass(gate_full(inp, run_target(inp, cuda)), f"split {shape} {dtype}")


@pytest.mark.parametrize("name,M,N", SPLIT_RECIPES)
def test_split_rows_recipes(cuda, name, M, N):
    inp = workloads.make_inputs(name, M=M, N=N)
    log(f"case split {name} recipe at M={M} N={N}")
    assert_pass(gate_full(inp, run_target(inp, cuda)), f"split {name} @ {M}x{N}")


@pytest.mark.parametrize("dtype,N", [(torch.float32, 1), (torch.bfloat16, 1), (torch.float16, 2),
                                     (torch.float32, 65536), (torch.float32, 65535),
                                     (torch.bfloat16, 65535), (torch.float16, 32769),
                                     (torch.bfloat16, 16385)])
def test_edge_shapes(cuda, dtype, N):
    M = 5
    inp = workloads.make_tile_case((M, N), dtype, 17)
    log(f"case edge {dtype} N={N}")
    assert_pass(gate_full(inp, run_target(inp, cuda)), f"edge {dtype} N={N}")


def test_m_zero(cuda):
    x = torch.empty((0, 64), device=cuda, dtype=torch.bfloat16)
    w = torch.ones(64, device=cuda, dtype=torch.bfloat16)
    y, r = rn.fwd(x, w)
    dx, dg = rn.bwd(x, x, w, r, poison=True)
    torch.cuda.synchronize()
    assert y.shape == (0, 64) and dx.shape == (0, 64)
    assert torch.equal(dg.cpu(), torch.zeros(64))


# Rows over 16384 elements that no full-width kernel takes (odd N, narrow
# alignment, float32 backward rows over 128 KiB) run the split kernels;
# several rows per row block, P set by the natural vector width.
GENERIC_SPLIT = [((300, 20001), torch.float16, "bwd_split", "fwd_split"),
                 ((40, 40000), torch.float32, "bwd_split", "fwd_rows"),
                 ((64, 65535), torch.bfloat16, "bwd_split", "fwd_split")]


@pytest.mark.parametrize("shape,dtype,bwd_kernel,fwd_kernel", GENERIC_SPLIT)
def test_generic_long_rows_take_split(cuda, shape, dtype, bwd_kernel, fwd_kernel):
    M, N = shape
    assert rn.rmsnorm_query_plan(M, N, dtype, which=rn.PASS_BWD_ROWS)["kernel_name"] == bwd_kernel
    assert rn.rmsnorm_query_plan(M, N, dtype, which=rn.PASS_FWD)["kernel_name"] == fwd_kernel
    inp = workloads.make_tile_case(shape, dtype, 19)
    log(f"case generic long rows {shape} {dtype}")
    assert_pass(gate_full(inp, run_target(inp, cuda)), f"generic long rows {shape} {dtype}")


def test_full_size_sampled_fp32_long_rows(cuda):
    """c4's recipe in float32 (2048 x 65536: 256 KiB rows, the split
    backward), sampled rows and dgamma columns."""
    inp = workloads.make_inputs("c4", dtype=torch.float32)
    log("case c4 recipe in float32 full size generated")
    out = run_target(inp, cuda)
    log("case c4 float32 device run done")
    rows = sample_rows(inp, 256)
    cols = sample_cols(inp["N"], 64)
    assert_pass(gate_sampled(inp, out, rows, cols), "c4 float32 full size, sampled")
    for k in ("y", "dx", "rstd", "dgamma"):
        assert not torch.isnan(out[k]).any(), f"{k} has unwritten (NaN) elements"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("M,N", [(33, 4096), (9, 40000)])
def test_misaligned_pointers(cuda, dtype, M, N):
    """Buffers starting one element past an aligned address: narrower vectors
    (generic kernels, or the split kernels for rows over 16384)."""
    inp = workloads.make_inputs("c2", M=M, N=N, dtype=dtype)

    def shifted(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=cuda)
        v = buf[1:].view(t.shape)
        v.copy_(t.to(cuda))
        return v

    x, w, dy = shifted(inp["x"]), shifted(inp["w"]), shifted(inp["dy"])
    y = shifted(torch.full_like(inp["x"], float("nan")))
    rstd = torch.empty(M, device=cuda)
    rn.rmsnorm_fwd(x, w, inp["eps"], y, rstd)
    dx, dg = rn.bwd(dy, x, w, rstd, poison=True)
    torch.cuda.synchronize()
    out = {"y": y, "rstd": rstd, "dx": dx, "dgamma": dg}
    assert_pass(gate_full(inp, out), f"misaligned {dtype}")


def test_binding_rejects_bad_tensors(cuda):
    x = torch.randn(8, 64, device=cuda).to(torch.bfloat16)
    w = torch.ones(64, device=cuda, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        rn.fwd(x.t(), torch.ones(8, device=cuda, dtype=torch.bfloat16))  # non-contiguous
    with pytest.raises(ValueError):
        rn.fwd(x, w.float())                                            # dtype mismatch
    with pytest.raises(ValueError):
        rn.fwd(x.double(), w.double())                                  # unsupported dtype
    with pytest.raises(rn.RmsnormError):
        rn.fwd(x, w, eps=0.0)
    with pytest.raises(rn.RmsnormError):
        n = rn.MAX_N + 1
        rn.fwd(torch.empty(2, n, device=cuda, dtype=torch.bfloat16),
               torch.ones(n, device=cuda, dtype=torch.bfloat16))
