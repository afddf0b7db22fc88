"""Cast-after-norm entry points (include/rmsnorm_cast.h) on the host:
argument checks and plans, no device work.  Every call below is invalid in
exactly one way, so nothing is ever launched on the fake addresses."""
import ctypes
import os

import pytest

import backward_rmsnorm_fwd_amd as rn

pytestmark = pytest.mark.skipif(not os.path.exists(rn.library_path()),
                                reason="librmsnorm.so not built")

OK, ENULL, EDTYPE, ESHAPE, EEPS, EFLAGS, EWS, EALIGN, EOVL = 0, -1, -2, -3, -4, -5, -6, -7, -8
EARG, ESTRIDE = -10, -11
F32, F16, BF16 = 0, 1, 2
A = 0x10000000  # fake, 16-byte aligned "device" addresses; never dereferenced
S = 1 << 24


def lib():
    return rn.load_library()


def fwd_call(x=A, g=A + S, eps=1e-6, M=4, N=256, dtype=F32, out=BF16, flags=0, y=A + 2 * S,
             rstd=A + 3 * S, ldx=None, ldy=None):
    ldx = N if ldx is None else ldx
    ldy = N if ldy is None else ldy
    return lib().rmsnorm_cast_fwd(x, ldx, g, eps, M, N, dtype, out, flags, y, ldy, rstd, None)


@pytest.mark.parametrize("kw,code", [
    ({"dtype": BF16}, EDTYPE), ({"dtype": F16}, EDTYPE), ({"out": F32}, EDTYPE),
    ({"out": 3}, EDTYPE), ({"flags": 4}, EFLAGS),
    ({"N": 0}, ESHAPE), ({"N": (1 << 24) + 1}, ESHAPE), ({"M": -1}, ESHAPE),
    ({"eps": 0.0}, EEPS), ({"eps": float("inf")}, EEPS),
    ({"ldx": 255}, ESTRIDE), ({"ldy": 100}, ESTRIDE),
    ({"x": None}, ENULL), ({"g": None}, ENULL), ({"y": None}, ENULL), ({"rstd": None}, ENULL),
    ({"x": A + 2}, EALIGN),                 # float32 input on a 2-byte boundary
    ({"g": A + S + 2}, EALIGN), ({"y": A + 2 * S + 1}, EALIGN),
    ({"rstd": A + 3 * S + 2}, EALIGN),
    ({"y": A + 64}, EOVL),                  # y overlaps x
    ({"rstd": A + S + 8}, EOVL),            # rstd overlaps gamma
    ({"rstd": A + 2 * S + 16}, EOVL),       # rstd overlaps y
    # spans past the 2^57 address limit, y == x: a stride error, never a launch
    ({"M": 1 << 40, "N": 1, "ldx": 1 << 40, "ldy": 1 << 40, "y": A}, ESTRIDE),
    ({"M": 1 << 40, "N": 1, "ldx": 1 << 22, "ldy": 1 << 22, "y": A}, ESTRIDE),
])
def test_fwd_rejects(kw, code):
    assert fwd_call(**kw) == code


def test_fwd_m0_is_a_noop():
    assert fwd_call(M=0, x=None, g=None, y=None, rstd=None) == OK


def bwd_call(dy=A, x=A + S, g=A + 2 * S, rstd=A + 3 * S, M=4, N=256, dtype=F32, out=BF16,
             flags=0, dx=A + 4 * S, dg=A + 5 * S, ws=A + 6 * S, ws_bytes=None, lddy=None,
             ldx=None, lddx=None):
    if ws_bytes is None:
        ws_bytes = lib().rmsnorm_cast_bwd_workspace_bytes(M, N, dtype, out, flags)
    lddy = N if lddy is None else lddy
    ldx = N if ldx is None else ldx
    lddx = N if lddx is None else lddx
    return lib().rmsnorm_cast_bwd(dy, lddy, x, ldx, g, rstd, M, N, dtype, out, flags, dx, lddx,
                                  dg, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    ({"dtype": F16}, EDTYPE), ({"out": F32}, EDTYPE), ({"flags": 8}, EFLAGS),
    ({"N": (1 << 24) + 1}, ESHAPE), ({"lddx": 3}, ESTRIDE), ({"lddy": 255}, ESTRIDE),
    ({"dy": None}, ENULL), ({"x": None}, ENULL), ({"g": None}, ENULL), ({"rstd": None}, ENULL),
    ({"dx": None}, ENULL), ({"dg": None}, ENULL),
    ({"ws": None}, EWS), ({"ws_bytes": 16}, EWS), ({"ws": A + 6 * S + 8}, EALIGN),
    ({"dy": A + 1}, EALIGN), ({"dx": A + 4 * S + 2}, EALIGN), ({"x": A + S + 2}, EALIGN),
    ({"dx": A + 16}, EOVL),                 # dx overlaps dy
    ({"dx": A + S + 64}, EOVL),             # dx overlaps x
    ({"dg": A + 3 * S + 4}, EOVL),          # dgamma overlaps rstd
    ({"ws": A + 4 * S + 256}, EOVL),        # workspace overlaps dx
])
def test_bwd_rejects(kw, code):
    assert bwd_call(**kw) == code


def test_bwd_m0_still_needs_dgamma():
    assert bwd_call(M=0, dg=None, dy=None, x=None, g=None, rstd=None, dx=None, ws=None) == ENULL


def test_rows_and_reduce_reject():
    L = lib()
    ws_bytes = L.rmsnorm_cast_bwd_workspace_bytes(4, 256, F32, BF16, 0)
    assert L.rmsnorm_cast_bwd_rows(A, 256, A + S, 256, A + 2 * S, A + 3 * S, 4, 256, F32, F16,
                                   0, A + 4 * S, 256, None, ws_bytes, None) == EWS
    assert L.rmsnorm_cast_bwd_reduce(A, ws_bytes, 4, 256, BF16, BF16, 0, A + S, None) == EDTYPE
    assert L.rmsnorm_cast_bwd_reduce(A, 8, 4, 256, F32, BF16, 0, A + S, None) == EWS


@pytest.mark.parametrize("out", ["bfloat16", "float16"])
def test_plans_are_the_float32_row_resident_plans(out):
    """The cast path takes LayerNorm's float32 row-resident plan: geometry,
    P and workspace are those of a float32 input (the narrow operands ride
    along at half the bytes per lane)."""
    import torch
    od = getattr(torch, out)
    for n in (1, 128, 1000, 4096, 4097, 5120, 16384):
        for m in (1, 1000, 32768):
            for which in (rn.PASS_FWD, rn.PASS_BWD_ROWS, rn.PASS_BWD_REDUCE):
                for align in (16, 8, 4):
                    c = rn.rmsnorm_cast_query_plan(m, n, od, which=which, align_bytes=align)
                    b = rn.layernorm_query_plan(m, n, torch.float32, which=which,
                                                align_bytes=align)
                    for k in ("vec", "threads_per_row", "block_threads", "chunks", "grid",
                              "partials", "lds_bytes"):
                        assert c[k] == b[k], (n, m, which, k)
                    want = {rn.PASS_FWD: "cast_fwd", rn.PASS_BWD_ROWS: "cast_bwd"}.get(which)
                    if want:
                        assert c["kernel_name"] == want
                        assert c["vec"] * 4 <= align
            P = rn.rmsnorm_cast_query_plan(m, n, od, which=rn.PASS_BWD_ROWS)["partials"]
            assert rn.rmsnorm_cast_bwd_workspace_bytes(m, n, od) == P * n * 4


def test_query_plan_rejects():
    L = lib()
    p = rn.Plan()
    assert L.rmsnorm_cast_query_plan(4, 256, F32, BF16, 0, 7, 16, ctypes.byref(p)) == EARG
    assert L.rmsnorm_cast_query_plan(4, 256, F32, BF16, 0, 0, 3, ctypes.byref(p)) == EARG
    assert L.rmsnorm_cast_query_plan(4, 256, BF16, BF16, 0, 0, 16, ctypes.byref(p)) == EDTYPE
    assert L.rmsnorm_cast_query_plan(4, (1 << 24) + 1, F32, F16, 0, 0, 16,
                                     ctypes.byref(p)) == ESHAPE
    assert L.rmsnorm_cast_query_plan(4, 256, F32, F16, 0, 0, 16, None) == ENULL
    assert L.rmsnorm_cast_bwd_workspace_bytes(0, 256, F32, BF16, 0) == 0
    assert L.rmsnorm_cast_bwd_workspace_bytes(4, 256, F32, F32, 0) == 0


@pytest.mark.parametrize("out", ["bfloat16", "float16"])
@pytest.mark.parametrize("M,N", [(33, 16385), (7, 16388), (2048, 65536), (2, 1 << 24),
                                 (100000, 20000)])
def test_split_plan(out, M, N):
    """Rows over the row-resident limit take RMSNorm's float32 split
    geometry: 16 KiB segments of x (4096 elements), P and the workspace of a
    float32 RMSNorm split; the access width keeps the narrow y and dy within
    the layout's alignment."""
    import torch
    od = getattr(torch, out)
    nseg = -(-N // 4096)
    f = rn.rmsnorm_cast_query_plan(M, N, od, which=rn.PASS_FWD)
    b = rn.rmsnorm_cast_query_plan(M, N, od, which=rn.PASS_BWD_ROWS)
    assert f["kernel_name"] == "cast_fwd_split" and b["kernel_name"] == "cast_bwd_split"
    for p in (f, b):
        assert p["segments"] == nseg and p["chunks"] * p["vec"] * 4 == 64
    ln = rn.layernorm_query_plan(M, N, torch.float32, which=rn.PASS_BWD_ROWS)
    assert (b["grid"], b["partials"]) == (ln["grid"], ln["partials"])
    P = b["partials"]
    r4 = lambda v: -(-v // 4) * 4  # noqa: E731
    assert rn.rmsnorm_cast_bwd_workspace_bytes(M, N, od) == 4 * (r4(P * N) + r4(M * nseg)
                                                                + r4(M))
    for align in (16, 8, 4):
        p = rn.rmsnorm_cast_query_plan(M, N, od, which=rn.PASS_FWD, align_bytes=align)
        assert p["vec"] * 4 <= align and N % p["vec"] == 0
