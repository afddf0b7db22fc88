"""Fused residual-add RMSNorm entry points (include/rmsnorm_add.h) on the
host: argument checks and plans, no device work.  Every call below is
invalid in exactly one way, so nothing is ever launched on the fake
addresses."""
import os

import pytest

import backward_rmsnorm_fwd_amd as rn

pytestmark = pytest.mark.skipif(not os.path.exists(rn.library_path()),
                                reason="librmsnorm.so not built")

OK, ENULL, EDTYPE, ESHAPE, EEPS, EFLAGS, EWS, EALIGN, EOVL = 0, -1, -2, -3, -4, -5, -6, -7, -8
ESTRIDE = -11
A = 0x10000000
S = 1 << 24


def lib():
    return rn.load_library()


def fwd_call(x=A, res=A + S, g=A + 2 * S, eps=1e-6, M=4, N=256, dtype=2, flags=0, y=A + 3 * S,
             h=A + 4 * S, rstd=A + 5 * S, ldr=None, ldh=None):
    ldr = N if ldr is None else ldr
    ldh = N if ldh is None else ldh
    return lib().rmsnorm_add_fwd(x, N, res, ldr, g, eps, M, N, dtype, flags, y, N, h, ldh, rstd,
                                 None)


@pytest.mark.parametrize("kw,code", [
    ({"dtype": 3}, EDTYPE), ({"flags": 4}, EFLAGS), ({"N": 0}, ESHAPE), ({"N": (1 << 24) + 1}, ESHAPE),
    ({"eps": -1.0}, EEPS), ({"ldr": 10}, ESTRIDE), ({"ldh": 255}, ESTRIDE),
    ({"x": None}, ENULL), ({"res": None}, ENULL), ({"g": None}, ENULL), ({"y": None}, ENULL),
    ({"h": None}, ENULL), ({"rstd": None}, ENULL),
    ({"res": A + S + 1}, EALIGN), ({"h": A + 4 * S + 1}, EALIGN),
    ({"h": A + 64}, EOVL),                # h overlaps x
    ({"h": A + S + 32}, EOVL),            # h overlaps res (in place is not accepted)
    ({"y": A + 4 * S + 8}, EOVL),         # y overlaps h
    ({"rstd": A + 2 * S}, EOVL),          # rstd overlaps gamma
    # spans past the 2^57 address limit, h == res: a stride error, never a launch
    ({"M": 1 << 40, "N": 1, "ldr": 1 << 40, "ldh": 1 << 40, "h": A + S}, ESTRIDE),
    ({"M": 1 << 40, "N": 1, "ldr": 1 << 22, "ldh": 1 << 22, "h": A + S}, ESTRIDE),
])
def test_fwd_rejects(kw, code):
    assert fwd_call(**kw) == code


def test_fwd_m0_is_a_noop():
    assert fwd_call(M=0, x=None, res=None, g=None, y=None, h=None, rstd=None) == OK


def bwd_call(dy=A, dh=A + S, h=A + 2 * S, g=A + 3 * S, rstd=A + 4 * S, M=4, N=256, dtype=2,
             flags=0, dx=A + 5 * S, dg=A + 6 * S, ws=A + 7 * S, ws_bytes=None, lddh=None):
    if ws_bytes is None:
        ws_bytes = lib().rmsnorm_add_bwd_workspace_bytes(M, N, dtype, flags)
    lddh = N if lddh is None else lddh
    return lib().rmsnorm_add_bwd(dy, N, dh, lddh, h, N, g, rstd, M, N, dtype, flags, dx, N, dg,
                                 ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    ({"dtype": 7}, EDTYPE), ({"flags": 8}, EFLAGS), ({"N": (1 << 24) + 1}, ESHAPE),
    ({"lddh": 3}, ESTRIDE),
    ({"dy": None}, ENULL), ({"h": None}, ENULL), ({"g": None}, ENULL), ({"rstd": None}, ENULL),
    ({"dx": None}, ENULL), ({"dg": None}, ENULL),
    ({"ws": None}, EWS), ({"ws_bytes": 8}, EWS), ({"ws": A + 7 * S + 8}, EALIGN),
    ({"dh": A + S + 1}, EALIGN),
    ({"dx": A + S + 16}, EOVL),           # dx overlaps dh
    ({"dx": A + 2 * S}, EOVL),            # dx overlaps h
    ({"dg": A + 4 * S + 4}, EOVL),        # dgamma overlaps rstd
    ({"ws": A + 5 * S + 512}, EOVL),      # workspace overlaps dx
])
def test_bwd_rejects(kw, code):
    assert bwd_call(**kw) == code


@pytest.mark.parametrize("dt", [0, 1, 2])
def test_plans_follow_the_row_resident_plan(dt):
    for n in (1, 128, 1000, 4096, 4097, 5120, 16384):
        for m in (1, 1000, 32768):
            for which in (rn.PASS_FWD, rn.PASS_BWD_ROWS, rn.PASS_BWD_REDUCE):
                a = rn.rmsnorm_add_query_plan(m, n, dt, which=which)
                b = rn.layernorm_query_plan(m, n, dt, which=which)
                keys = ["vec", "threads_per_row", "block_threads", "chunks", "partials",
                        "lds_bytes"] + ([] if which == rn.PASS_FWD else ["grid"])
                lnb = rn.layernorm_query_plan(m, n, dt, which=rn.PASS_BWD_ROWS)
                if which != rn.PASS_FWD and lnb["kernel_name"] == "ln_bwd_rows":
                    # LayerNorm's own two-rows backward (and its P) for 4-8 KiB
                    # rows; the fused add keeps the row-resident plan
                    keys = ["vec", "block_threads", "grid"] if which == rn.PASS_BWD_REDUCE else []
                    assert a["partials"] == min(512, m)
                for k in keys:
                    assert a[k] == b[k], (n, m, which, k)
                if which == rn.PASS_FWD:
                    # One row step per workgroup: G row groups x R rows, where a
                    # row group takes two rows per step when their operands fit
                    # in 16 VGPRs (8 in workgroups over 256 threads); LayerNorm
                    # reads one row operand, the fused add two.
                    es = 4 if dt == 0 else 2
                    G = b["block_threads"] // b["threads_per_row"]
                    maxc = 1 << (b["chunks"] - 1).bit_length()
                    regs = -(-(b["vec"] * es) // 4)
                    lim = 16 if b["block_threads"] == 256 else 8
                    cap = 65536 * 256 // b["block_threads"]
                    for plan, mats in ((b, 1), (a, 2)):
                        R = 2 if maxc * regs * mats <= lim else 1
                        assert plan["grid"] == min(-(-m // (G * R)), cap), (n, m, mats)
                want = {rn.PASS_FWD: "add_fwd", rn.PASS_BWD_ROWS: "add_bwd"}.get(which)
                if want:
                    assert a["kernel_name"] == want
            P = rn.rmsnorm_add_query_plan(m, n, dt, which=rn.PASS_BWD_ROWS)["partials"]
            assert rn.rmsnorm_add_bwd_workspace_bytes(m, n, dt) == P * n * 4


def _ceil(a, b):
    return -(-a // b)


def _long(N, es, align=16):
    """Full-width rows of 16 to 128 KiB over 16384 elements (RMSNorm's
    long-row range: 5 to 16 chunks of 8 KiB per 512-thread row)."""
    vec = 16 // es
    return N > 16384 and align >= 16 and N % vec == 0 and 5 <= _ceil(N // vec, 512) <= 16


@pytest.mark.parametrize("M,N,dt", [(33, 16385, 2), (5, 16386, 1), (7, 16388, 0),
                                    (2, 1 << 24, 2), (2048, 65536, 2), (100000, 20000, 1),
                                    (4096, 65537, 0), (700, 16400, 2), (9, 32768, 0),
                                    (9, 40000, 0)])
def test_long_and_split_plans(M, N, dt):
    """Rows over the row-resident limit: full-width rows of up to 128 KiB
    take RMSNorm's long-row kernels (one 512-thread workgroup per row, P =
    min(M, 256)); other rows, and those under a narrower alignment, take
    RMSNorm's split geometry on the same P.  The workspace has the split
    layout ([P, N] partials, per-(row, segment) sums, per-row
    coefficients) either way."""
    es = 4 if dt == 0 else 2
    nseg = _ceil(N * es, 16384)
    long_rows = _long(N, es)
    P = min(M, 256) if long_rows else \
        max(1, min(M, max(_ceil(M, 16), _ceil(1024, nseg)), ((1 << 24) - 1) // nseg))
    for align in (16, 8, 4, 2):
        if es == 4 and align < 4:
            continue
        f = rn.rmsnorm_add_query_plan(M, N, dt, which=rn.PASS_FWD, align_bytes=align)
        b = rn.rmsnorm_add_query_plan(M, N, dt, which=rn.PASS_BWD_ROWS, align_bytes=align)
        assert b["partials"] == P
        if _long(N, es, align):
            assert f["kernel_name"] == "add_fwd_long" and b["kernel_name"] == "add_bwd_long"
            ch = _ceil(N // (16 // es), 512)
            for p in (f, b):
                assert (p["threads_per_row"], p["block_threads"], p["chunks"]) == (512, 512, ch)
            assert b["grid"] == P and b["lds_bytes"] == N * es
            assert f["grid"] == min(M, 1 << 20)
        else:
            assert f["kernel_name"] == "add_fwd_split" and b["kernel_name"] == "add_bwd_split"
            for p in (f, b):
                assert p["segments"] == nseg and p["block_threads"] == 256
                assert p["chunks"] * p["vec"] * es == 64 and p["grid"] % nseg == 0
            assert b["grid"] == P * nseg
            # the forward keeps no column sums: one row per block
            assert f["grid"] // nseg == max(1, min(M, ((1 << 24) - 1) // nseg))
    r4 = lambda v: _ceil(v, 4) * 4  # noqa: E731
    assert rn.rmsnorm_add_bwd_workspace_bytes(M, N, dt) == 4 * (r4(P * N) + r4(M * nseg) + r4(M))
    assert rn.rmsnorm_add_query_plan(M, N, dt, which=rn.PASS_BWD_REDUCE)["partials"] == P
    if long_rows and N <= 65536:
        r = rn.rmsnorm_query_plan(M, N, dt, which=rn.PASS_BWD_ROWS)
        assert r["kernel_name"] == "bwd_long" and r["partials"] == P
