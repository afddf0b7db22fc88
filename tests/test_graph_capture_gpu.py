"""The C ABI under HIP graph capture (torch.cuda.CUDAGraph): a forward +
backward step of RMSNorm (with a caller workspace and with the
allocation-free backward), of LayerNorm, of the fused residual add and of
the fused output cast, captured once and replayed
several times on new input data, with eager work and synchronisation
between the replays.  The library enqueues kernels only (no allocation, no
memset, no host synchronisation), so every replay must give the same bits
as an eager call on the same data: the same kernels and plans run in both.

Only library calls are captured; the buffers are filled and poisoned with
NaN by eager work outside the graph."""
import pytest
import torch

import backward_rmsnorm_fwd_amd as rn
from backward_rmsnorm_fwd_amd import workloads
from parity import log

pytestmark = pytest.mark.gpu

EPS = 1e-6
# Row-resident (c2's shape class), the pipelined backward, long rows, split
# rows past 65536, and odd N over 16384 (split kernels with 2-byte accesses).
SHAPES = [((1024, 4096), torch.bfloat16), ((2048, 1024), torch.float16),
          ((40, 65536), torch.bfloat16), ((12, 131072), torch.float32),
          ((96, 20001), torch.float16)]


def _capture(step):
    """Warm the step up on a side stream, then capture it."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    return graph


def _inputs(shape, dtype, seeds):
    return [workloads.make_layernorm_tile_case(shape, dtype, s) for s in seeds]


@pytest.mark.parametrize("shape,dtype", SHAPES)
def test_rmsnorm_step_replays_match_eager(cuda, shape, dtype):
    M, N = shape
    data = _inputs(shape, dtype, (71, 72, 73))
    x = torch.empty(shape, dtype=dtype, device=cuda)
    dy, y, dx, dx2 = (torch.empty_like(x) for _ in range(4))
    w = torch.empty(N, dtype=dtype, device=cuda)
    rstd = torch.empty(M, device=cuda)
    dg, dg2 = torch.empty(N, device=cuda), torch.empty(N, device=cuda)
    ws = torch.empty(max(4, rn.rmsnorm_bwd_workspace_bytes(M, N, dtype)) // 4, device=cuda)
    noalloc = rn.rmsnorm_bwd_workspace_bytes(M, N, dtype) <= rn.NOALLOC_SCRATCH_BYTES

    def load(k):
        x.copy_(data[k]["x"])
        dy.copy_(data[k]["dy"])
        w.copy_(data[k]["w"])

    def step():
        rn.rmsnorm_fwd(x, w, EPS, y, rstd)
        rn.rmsnorm_bwd(dy, x, w, rstd, dx, dg, ws)
        if noalloc:
            rn.rmsnorm_bwd_noalloc(dy, x, w, rstd, dx2, dg2)

    load(0)
    graph = _capture(step)
    for rep in range(4):
        k = rep % len(data)
        load(k)
        for t in (y, dx, dx2):
            t.fill_(float("nan"))
        for t in (dg, dg2, rstd):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        log(f"case graph rmsnorm {shape} {dtype} replay {rep} data {k}")
        graph.replay()
        torch.cuda.synchronize()
        ye, re = rn.fwd(x, w, EPS)
        dxe, dge = rn.bwd(dy, x, w, re)
        torch.cuda.synchronize()
        assert torch.equal(y, ye) and torch.equal(rstd, re), rep
        assert torch.equal(dx, dxe) and torch.equal(dg, dge), rep
        if noalloc:
            assert torch.equal(dx2, dxe) and torch.equal(dg2, dge), rep


@pytest.mark.parametrize("shape,dtype", [((1024, 4096), torch.bfloat16),
                                         ((24, 40000), torch.bfloat16),
                                         ((96, 20001), torch.float16)])
def test_layernorm_step_replays_match_eager(cuda, shape, dtype):
    M, N = shape
    data = _inputs(shape, dtype, (81, 82))
    x = torch.empty(shape, dtype=dtype, device=cuda)
    dy, y, dx = (torch.empty_like(x) for _ in range(3))
    w = torch.empty(N, dtype=dtype, device=cuda)
    b = torch.empty(N, dtype=dtype, device=cuda)
    mean, rstd = torch.empty(M, device=cuda), torch.empty(M, device=cuda)
    dg, db = torch.empty(N, device=cuda), torch.empty(N, device=cuda)
    ws = torch.empty(max(4, rn.layernorm_bwd_workspace_bytes(M, N, dtype)) // 4, device=cuda)

    def load(k):
        x.copy_(data[k]["x"])
        dy.copy_(data[k]["dy"])
        w.copy_(data[k]["w"])
        b.copy_(data[k]["b"])

    def step():
        rn.layernorm_fwd(x, w, b, EPS, y, mean, rstd)
        rn.layernorm_bwd(dy, x, w, mean, rstd, dx, dg, db, ws)

    load(0)
    graph = _capture(step)
    for rep in range(4):
        k = rep % len(data)
        load(k)
        for t in (y, dx, mean, rstd, dg, db):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        log(f"case graph layernorm {shape} {dtype} replay {rep} data {k}")
        graph.replay()
        torch.cuda.synchronize()
        ye, me, re = rn.ln_fwd(x, w, b, EPS)
        dxe, dge, dbe = rn.ln_bwd(dy, x, w, me, re)
        torch.cuda.synchronize()
        assert torch.equal(y, ye) and torch.equal(mean, me) and torch.equal(rstd, re), rep
        assert torch.equal(dx, dxe) and torch.equal(dg, dge) and torch.equal(db, dbe), rep


@pytest.mark.parametrize("shape,dtype", [((1024, 4096), torch.bfloat16),
                                         ((40, 65536), torch.bfloat16),
                                         ((96, 20001), torch.float16)])
def test_fused_add_step_replays_match_eager(cuda, shape, dtype):
    """The residual add fused with RMSNorm: row-resident, long rows (the
    long-row kernels with the add) and odd rows past 16384 (split kernels)."""
    M, N = shape
    data = _inputs(shape, dtype, (91, 92))
    x = torch.empty(shape, dtype=dtype, device=cuda)
    res, dy, dh, y, h, dx = (torch.empty_like(x) for _ in range(6))
    w = torch.empty(N, dtype=dtype, device=cuda)
    rstd, dg = torch.empty(M, device=cuda), torch.empty(N, device=cuda)
    ws = torch.empty(max(4, rn.rmsnorm_add_bwd_workspace_bytes(M, N, dtype)) // 4, device=cuda)

    def load(k):
        x.copy_(data[k]["x"])
        res.copy_(data[k]["dy"])  # any second operand of the same shape
        dy.copy_(data[k]["dy"].flip(0))
        dh.copy_(data[k]["x"].flip(0))
        w.copy_(data[k]["w"])

    def step():
        rn.rmsnorm_add_fwd(x, res, w, EPS, y, h, rstd)
        rn.rmsnorm_add_bwd(dy, dh, h, w, rstd, dx, dg, ws)

    load(0)
    graph = _capture(step)
    for rep in range(4):
        k = rep % len(data)
        load(k)
        for t in (y, h, dx, rstd, dg):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        log(f"case graph add {shape} {dtype} replay {rep} data {k}")
        graph.replay()
        torch.cuda.synchronize()
        ye, he, re = rn.add_fwd(x, res, w, EPS)
        dxe, dge = rn.add_bwd(dy, dh, he, w, re)
        torch.cuda.synchronize()
        assert torch.equal(y, ye) and torch.equal(h, he) and torch.equal(rstd, re), rep
        assert torch.equal(dx, dxe) and torch.equal(dg, dge), rep


@pytest.mark.parametrize("shape,out_dtype", [((1024, 4096), torch.bfloat16),
                                             ((12, 131072), torch.float16)])
def test_cast_step_replays_match_eager(cuda, shape, out_dtype):
    """RMSNorm with its output cast: row-resident and split rows."""
    M, N = shape
    data = _inputs(shape, torch.float32, (93, 94))
    x = torch.empty(shape, dtype=torch.float32, device=cuda)
    dx = torch.empty_like(x)
    y = torch.empty(shape, dtype=out_dtype, device=cuda)
    dy = torch.empty_like(y)
    w = torch.empty(N, device=cuda)
    rstd, dg = torch.empty(M, device=cuda), torch.empty(N, device=cuda)
    ws = torch.empty(max(4, rn.rmsnorm_cast_bwd_workspace_bytes(M, N, out_dtype)) // 4,
                     device=cuda)

    def load(k):
        x.copy_(data[k]["x"])
        dy.copy_(data[k]["dy"])
        w.copy_(data[k]["w"])

    def step():
        rn.rmsnorm_cast_fwd(x, w, EPS, y, rstd)
        rn.rmsnorm_cast_bwd(dy, x, w, rstd, dx, dg, ws)

    load(0)
    graph = _capture(step)
    for rep in range(4):
        k = rep % len(data)
        load(k)
        for t in (dx, rstd, dg):
            t.fill_(float("nan"))
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        log(f"case graph cast {shape} {out_dtype} replay {rep} data {k}")
        graph.replay()
        torch.cuda.synchronize()
        ye, re = rn.cast_fwd(x, w, out_dtype, EPS)
        dxe, dge = rn.cast_bwd(dy, x, w, re)
        torch.cuda.synchronize()
        assert torch.equal(y, ye) and torch.equal(rstd, re), rep
        assert torch.equal(dx, dxe) and torch.equal(dg, dge), rep
