"""rmsnorm_bwd_noalloc (the backward with its dgamma partials in the
library's own device buffer) against rmsnorm_bwd (caller workspace), through
the C ABI on the GPU.

Both entry points run the same kernels with the same plan, so dx and dgamma
must be bitwise identical.  Two calls in a row on the shared buffer, the
second smaller than the first, show that the leftovers of a larger call do
not reach a smaller one; the smaller call is also gated against the oracle.
"""
import pytest
import torch

import backward_rmsnorm_fwd_amd as rn
from backward_rmsnorm_fwd_amd import workloads
from parity import assert_pass, gate_full, log

pytestmark = pytest.mark.gpu

# (name, M, N, dtype, offset, seed): the first of each pair needs more partial
# sums than the second.  2048 x 65536 bf16 needs 64 MiB of partial sums plus
# the split plan's row sums (any layout of rows over 16384 may run them).
PAIRS = [
    (("c4", 2048, 65536, torch.bfloat16, False, 1), ("c1a", None, None, None, None, None)),
    (("c2", 32768, 4096, torch.bfloat16, False, 2), ("tile", 513, 5120, torch.bfloat16, True, 3)),
    (("c3", 8192, 1024, torch.float16, False, 4), ("tile", 37, 2048, torch.float32, False, 5)),
    (("tile", 64, 200000, torch.float32, False, 6), ("tile", 9, 70000, torch.bfloat16, False, 7)),
]


def _inputs(spec):
    name, M, N, dtype, offset, seed = spec
    if name == "tile":
        inp = workloads.make_tile_case((M, N), dtype, seed)
        if offset:
            inp["offset"] = True
        return inp
    return workloads.make_inputs(name, M=M, N=N)


def _both(inp, dev):
    x, w, dy = (inp[k].to(dev) for k in ("x", "w", "dy"))
    off = inp["offset"]
    y, rstd = rn.fwd(x, w, inp["eps"], off)
    M, N = x.shape[0], x.shape[-1]
    dx_a = torch.full_like(x, float("nan"))
    dg_a = torch.full((N,), float("nan"), device=dev, dtype=torch.float32)
    dx_b = torch.full_like(x, float("nan"))
    dg_b = torch.full((N,), float("nan"), device=dev, dtype=torch.float32)
    nbytes = rn.rmsnorm_bwd_workspace_bytes(M, N, x.dtype, off)
    assert nbytes <= rn.NOALLOC_SCRATCH_BYTES
    ws = torch.full((max(nbytes, 4) // 4,), float("nan"), device=dev, dtype=torch.float32)
    rn.rmsnorm_bwd(dy, x, w, rstd, dx_a, dg_a, ws, off)
    rn.rmsnorm_bwd_noalloc(dy, x, w, rstd, dx_b, dg_b, off)
    torch.cuda.synchronize()
    return {"y": y, "rstd": rstd, "dx": dx_b, "dgamma": dg_b}, (dx_a, dg_a), (dx_b, dg_b)


@pytest.mark.parametrize("big,small", PAIRS, ids=[f"{a[0]}-{a[1]}x{a[2]}" for a, _ in PAIRS])
def test_noalloc_matches_workspace_entry_point(cuda, big, small):
    for step, spec in (("first", big), ("second", small)):
        inp = _inputs(spec)
        shape = tuple(inp["x"].shape)
        log(f"noalloc {step} call: {spec[0]} {shape} {inp['x'].dtype} offset={inp['offset']}")
        out, (dx_a, dg_a), (dx_b, dg_b) = _both(inp, cuda)
        bits = torch.int32 if dx_a.dtype == torch.float32 else torch.int16
        assert torch.equal(dx_a.view(bits), dx_b.view(bits))
        assert torch.equal(dg_a.view(torch.int32), dg_b.view(torch.int32))
        if step == "second":
            assert_pass(gate_full(inp, {k: v for k, v in out.items()}), f"noalloc {spec[0]}")


def test_noalloc_rejects_shapes_beyond_its_buffer(cuda):
    # 32 rows of 2^24 float32 need two partial rows of 64 MiB plus the split
    # plan's row sums: more than the buffer, so the call is refused before
    # anything runs.
    M, N = 32, 1 << 24
    assert rn.rmsnorm_bwd_workspace_bytes(M, N, torch.float32) > rn.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M, N), device=cuda)
    dy, dx = torch.zeros_like(x), torch.zeros_like(x)
    w = torch.ones(N, device=cuda)
    rstd = torch.ones(M, device=cuda)
    dg = torch.zeros(N, device=cuda)
    with pytest.raises(RuntimeError, match="workspace"):
        rn.rmsnorm_bwd_noalloc(dy, x, w, rstd, dx, dg)


def test_noalloc_m0_writes_zero_dgamma(cuda):
    x = torch.empty((0, 4096), device=cuda, dtype=torch.bfloat16)
    w = torch.ones(4096, device=cuda, dtype=torch.bfloat16)
    dg = torch.full((4096,), float("nan"), device=cuda)
    rn.rmsnorm_bwd_noalloc(x, x, w, torch.empty(0, device=cuda), torch.empty_like(x), dg)
    torch.cuda.synchronize()
    assert torch.equal(dg, torch.zeros_like(dg))
