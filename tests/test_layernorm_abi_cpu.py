"""LayerNorm entry points (include/layernorm.h) on the host: argument checks
and launch plans, no device work.  Every call below is invalid in exactly
one way, so nothing is ever launched on the fake addresses."""
import ctypes

import pytest

import backward_rmsnorm_fwd_amd as rn

pytestmark = pytest.mark.skipif(not __import__("os").path.exists(rn.library_path()),
                                reason="librmsnorm.so not built")

OK, ENULL, EDTYPE, ESHAPE, EEPS, EFLAGS, EWS, EALIGN, EOVL = 0, -1, -2, -3, -4, -5, -6, -7, -8
EARG, ESTRIDE = -10, -11
A = 0x10000000  # fake, 16-byte aligned "device" addresses; never dereferenced
S = 1 << 24     # spacing between the fake buffers


def lib():
    return rn.load_library()


def fwd_call(x=A, ldx=None, g=A + S, b=A + 2 * S, eps=1e-5, M=4, N=256, dtype=2, flags=0,
             y=A + 3 * S, ldy=None, mean=A + 4 * S, rstd=A + 5 * S):
    ldx = N if ldx is None else ldx
    ldy = N if ldy is None else ldy
    return lib().layernorm_fwd(x, ldx, g, b, eps, M, N, dtype, flags, y, ldy, mean, rstd, None)


@pytest.mark.parametrize("kw,code", [
    ({"dtype": 3}, EDTYPE), ({"flags": 1}, EFLAGS), ({"flags": 4}, EFLAGS),
    ({"N": 0}, ESHAPE), ({"N": (1 << 24) + 1}, ESHAPE), ({"M": -1}, ESHAPE),
    ({"M": 1 << 40, "N": 65537}, ESHAPE),                 # M * N above 2^46
    ({"eps": 0.0}, EEPS), ({"eps": float("nan")}, EEPS),
    ({"ldx": 255}, ESTRIDE), ({"ldy": 100}, ESTRIDE),
    ({"x": None}, ENULL), ({"g": None}, ENULL), ({"y": None}, ENULL),
    ({"mean": None}, ENULL), ({"rstd": None}, ENULL),
    ({"x": A + 1}, EALIGN), ({"b": A + 2 * S + 1}, EALIGN), ({"mean": A + 4 * S + 2}, EALIGN),
    ({"y": A + 64}, EOVL),                  # y overlaps x
    ({"mean": A + S + 8}, EOVL),            # mean overlaps gamma
    ({"rstd": A + 2 * S + 4}, EOVL),        # rstd overlaps beta
    ({"rstd": A + 4 * S + 8}, EOVL),        # rstd overlaps mean
    # spans past the 2^57 address limit ((M - 1) * pitch passes 2^63 at the
    # first two pitches), y == x: a stride error, never a launch
    ({"M": 1 << 40, "N": 1, "ldx": 1 << 40, "ldy": 1 << 40, "y": A}, ESTRIDE),
    ({"M": 1 << 40, "N": 1, "ldx": 1 << 22, "ldy": 1 << 22, "y": A}, ESTRIDE),
    ({"M": 1 << 40, "N": 1, "ldx": 1 << 30}, ESTRIDE),
])
def test_fwd_rejects(kw, code):
    assert fwd_call(**kw) == code


def test_fwd_m0_is_a_noop():
    assert fwd_call(M=0, x=None, g=None, b=None, y=None, mean=None, rstd=None) == OK


def bwd_call(dy=A, x=A + S, g=A + 2 * S, mean=A + 3 * S, rstd=A + 4 * S, M=4, N=256,
             dtype=2, flags=0, dx=A + 5 * S, dg=A + 6 * S, db=A + 7 * S, ws=A + 8 * S,
             ws_bytes=None, lddy=None, ldx=None, lddx=None):
    if ws_bytes is None:
        ws_bytes = lib().layernorm_bwd_workspace_bytes(M, N, dtype, flags)
    lddy = N if lddy is None else lddy
    ldx = N if ldx is None else ldx
    lddx = N if lddx is None else lddx
    return lib().layernorm_bwd(dy, lddy, x, ldx, g, mean, rstd, M, N, dtype, flags, dx, lddx,
                               dg, db, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    ({"dtype": 5}, EDTYPE), ({"flags": 1}, EFLAGS), ({"N": (1 << 24) + 1}, ESHAPE),
    ({"lddx": 3}, ESTRIDE),
    ({"dy": None}, ENULL), ({"x": None}, ENULL), ({"g": None}, ENULL), ({"mean": None}, ENULL),
    ({"rstd": None}, ENULL), ({"dx": None}, ENULL), ({"dg": None}, ENULL),
    ({"ws": None}, EWS), ({"ws_bytes": 16}, EWS),
    ({"ws": A + 8 * S + 4}, EALIGN), ({"dy": A + 1}, EALIGN), ({"db": A + 7 * S + 2}, EALIGN),
    ({"dx": A + 16}, EOVL),                 # dx overlaps dy
    ({"dg": A + 3 * S + 4}, EOVL),          # dgamma overlaps mean
    ({"db": A + 6 * S + 8}, EOVL),          # dbeta overlaps dgamma
    ({"ws": A + 5 * S + 256}, EOVL),        # workspace overlaps dx
])
def test_bwd_rejects(kw, code):
    assert bwd_call(**kw) == code


def test_bwd_m0_still_needs_dgamma():
    assert bwd_call(M=0, dg=None, dy=None, x=None, g=None, mean=None, rstd=None, dx=None,
                    ws=None) == ENULL


def _ceil(a, b):
    return -(-a // b)


def _bwd_rows(n, es, align):
    """Backward rows of 257 to 512 16-byte vectors with a 16-byte layout run
    the two-rows-per-workgroup kernel with x in LDS."""
    vec = 16 // es
    return align >= 16 and n % vec == 0 and 256 < n // vec <= 512


@pytest.mark.parametrize("dt", [0, 1, 2])
def test_plans_cover_rows(dt):
    """Every N gets a plan whose lanes cover the row with no empty chunk,
    within the register-slot caps, in workgroups of max(256, row lanes)
    threads; P does not
    depend on alignment; the workspace holds two [P, N] blocks."""
    es = 4 if dt == 0 else 2
    for n in list(range(1, 130)) + [255, 256, 257, 1000, 1024, 4095, 4096, 4097, 5120, 8191,
                                    8192, 8193, 12288, 16383, 16384]:
        for m in (1, 7, 1000, 262144):
            P = None
            for align in (16, 8, 4, 2):
                if es == 4 and align < 4:
                    continue
                for which, target in ((rn.PASS_FWD, lambda v: min(4, 32 // v)),
                                      (rn.PASS_BWD_ROWS, lambda v: min(8, 16 // v))):
                    p = rn.layernorm_query_plan(m, n, dt, which=which, align_bytes=align)
                    vec, tpr, ch = p["vec"], p["threads_per_row"], p["chunks"]
                    assert n % vec == 0 and vec * es <= align
                    assert tpr * ch * vec >= n > tpr * (ch - 1) * vec
                    rows = which == rn.PASS_BWD_ROWS and _bwd_rows(n, es, align)
                    if rows:
                        assert p["kernel_name"] == "ln_bwd_rows"
                        assert (tpr, ch, p["block_threads"], p["x_in_lds"]) == (256, 2, 512, 1)
                        assert p["lds_bytes"] == max(2 * n * es, 2 * tpr * vec * 4)
                    else:
                        assert p["kernel_name"] == ("ln_fwd" if which == rn.PASS_FWD
                                                    else "ln_bwd")
                        assert p["block_threads"] == max(256, tpr) and 64 <= tpr <= 1024
                        cap = max(target(vec), 16 // vec)
                        assert ch <= cap
                    if which == rn.PASS_BWD_ROWS:
                        if P is None:
                            P = p["partials"]
                        assert p["partials"] == P == p["grid"]
                        bt = p["block_threads"]
                        if not rows:
                            assert p["lds_bytes"] == (0 if tpr == bt else bt * vec * 4)
            base = rn.layernorm_query_plan(m, n, dt, which=rn.PASS_BWD_ROWS)
            assert P == min(512, _ceil(m, base["block_threads"] // base["threads_per_row"]))
            assert rn.layernorm_bwd_workspace_bytes(m, n, dt) == 2 * P * n * 4
            red = rn.layernorm_query_plan(m, n, dt, which=rn.PASS_BWD_REDUCE)
            assert red["partials"] == P


def test_query_plan_rejects():
    L = lib()
    p = rn.Plan()
    assert L.layernorm_query_plan(4, 256, 2, 0, 7, 16, ctypes.byref(p)) == EARG
    assert L.layernorm_query_plan(4, 256, 2, 1, 0, 16, ctypes.byref(p)) == EFLAGS
    assert L.layernorm_query_plan(4, (1 << 24) + 1, 2, 0, 0, 16, ctypes.byref(p)) == ESHAPE
    assert L.layernorm_query_plan(4, 256, 2, 0, 0, 16, None) == ENULL
    assert rn.layernorm_bwd_workspace_bytes(0, 256, 2) == 0
    assert rn.layernorm_bwd_workspace_bytes(4, (1 << 24) + 1, 2) == 0
    assert rn.layernorm_bwd_workspace_bytes(0, 1 << 20, 2) == 0


@pytest.mark.parametrize("dt,n,tpr,ch", [(2, 5120, 320, 2), (1, 5120, 320, 2), (0, 5120, 320, 4),
                                         (1, 12288, 768, 2), (2, 4096, 256, 2), (0, 16384, 1024, 4)])
def test_backward_exact_fit(dt, n, tpr, ch):
    """Rows wider than four wavefronts whose 64-lane sweeps the power-of-two
    plan would leave partly idle take the fewest wavefronts (over four) that
    divide them exactly; the forward keeps its power-of-two plan."""
    p = rn.layernorm_query_plan(65536, n, dt, which=rn.PASS_BWD_ROWS)
    block = 512 if _bwd_rows(n, 4 if dt == 0 else 2, 16) else max(256, tpr)
    assert (p["threads_per_row"], p["chunks"], p["block_threads"]) == (tpr, ch, block)
    assert p["threads_per_row"] * p["chunks"] * p["vec"] == n
    a = rn.rmsnorm_add_query_plan(65536, n, dt, which=rn.PASS_BWD_ROWS)
    assert (a["threads_per_row"], a["chunks"]) == (tpr, ch)
    f = rn.layernorm_query_plan(65536, 5120, 2, which=rn.PASS_FWD)
    assert (f["threads_per_row"], f["chunks"], f["block_threads"]) == (256, 3, 256)


def _long_fwd(N, es, align=16):
    """Full-width forward rows over 16384 of at most 8 chunks per lane over
    16 wavefronts stay row-resident."""
    vec = 16 // es
    return N > 16384 and align >= 16 and N % vec == 0 and N // vec <= 8192


def _check_long_fwd(f, M, N, es):
    vec = 16 // es
    ch = _ceil(N // vec, 1024)
    assert f["kernel_name"] == "ln_fwd" and f["vec"] == vec
    assert (f["threads_per_row"], f["block_threads"], f["chunks"]) == (1024, 1024, ch)
    assert f["weight_in_regs"] == (1 if ch <= 4 else 0)
    assert f["grid"] == min(M, 16384)


@pytest.mark.parametrize("M,N,dt", [(33, 16385, 2), (5, 16386, 1), (7, 16388, 0),
                                    (2, 1 << 24, 2), (261, 98304, 2), (100000, 20000, 1),
                                    (1, 1 << 24, 0), (4096, 65537, 0), (8, 32768, 2)])
def test_split_plan(M, N, dt):
    """Rows longer than the row-resident limit: the RMSNorm split geometry
    (16 KiB segments, one 256-thread workgroup per (row block, segment), the
    same P); the workspace holds the two [P, N] column blocks, three sums per
    (row, segment) and three coefficients per row, each from a 16-byte
    boundary."""
    es = 4 if dt == 0 else 2
    nseg = _ceil(N * es, 16384)
    f = rn.layernorm_query_plan(M, N, dt, which=rn.PASS_FWD)
    b = rn.layernorm_query_plan(M, N, dt, which=rn.PASS_BWD_ROWS)
    assert b["kernel_name"] == "ln_bwd_split"
    if _long_fwd(N, es):
        _check_long_fwd(f, M, N, es)
        f = rn.layernorm_query_plan(M, N, dt, which=rn.PASS_FWD, align_bytes=8)
    assert f["kernel_name"] == "ln_fwd_split"
    rf = rn.rmsnorm_query_plan(M, max(N, 65537), dt, which=rn.PASS_FWD, align_bytes=8)
    for p in (f, b):
        assert p["segments"] == nseg and p["block_threads"] == 256
        assert p["threads_per_row"] == 256 * nseg
        assert p["grid"] % nseg == 0 and p["grid"] < 1 << 24
        assert p["chunks"] * p["vec"] * es == 64
        assert 1 <= p["grid"] // nseg <= M
    P = b["partials"]
    assert b["grid"] == P * nseg
    assert P == max(1, min(M, max(_ceil(M, 16), _ceil(1024, nseg)), ((1 << 24) - 1) // nseg))
    assert f["partials"] == 0
    assert f["grid"] // nseg == max(1, min(M, _ceil(2048, nseg), ((1 << 24) - 1) // nseg))
    if N > 65536:
        assert f["segments"] == rf["segments"]
    r4 = lambda v: _ceil(v, 4) * 4  # noqa: E731
    assert rn.layernorm_bwd_workspace_bytes(M, N, dt) == 4 * (r4(2 * P * N) + r4(3 * M * nseg)
                                                             + r4(3 * M))
    red = rn.layernorm_query_plan(M, N, dt, which=rn.PASS_BWD_REDUCE)
    assert red["partials"] == P


def test_split_plan_boundary_and_row_room():
    """16384 elements stay row-resident and 16385 split, in every dtype; a
    row of y has room for the forward's 16 bytes per segment plus nothing
    more (the mean's remainder reuses the first segment's slot)."""
    for dt in (0, 1, 2):
        es = 4 if dt == 0 else 2
        assert rn.layernorm_query_plan(3, 16384, dt)["kernel_name"] == "ln_fwd"
        assert rn.layernorm_query_plan(3, 16384, dt, which=rn.PASS_BWD_ROWS)["kernel_name"] \
            == "ln_bwd"
        for n in [16385, 16387, 16400, 24576, 65535, 65537, 131073, 999999, (1 << 24) - 1,
                  1 << 24]:
            for align in (16, 8, 4, 2):
                if es == 4 and align < 4:
                    continue
                p = rn.layernorm_query_plan(3, n, dt, which=rn.PASS_FWD, align_bytes=align)
                if _long_fwd(n, es, align):
                    _check_long_fwd(p, 3, n, es)
                    continue
                seg = 256 * p["chunks"] * p["vec"]
                assert p["kernel_name"] == "ln_fwd_split"
                assert seg * es == 16384 and n % p["vec"] == 0
                assert p["segments"] * seg >= n > (p["segments"] - 1) * seg
                assert 16 * p["segments"] <= n * es
