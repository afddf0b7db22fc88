"""Host-side tests of the C ABI: the library loads, exports every symbol the
header declares, and rejects invalid calls before any device work.

Every call here fails argument validation on the host (exactly one argument is
wrong in each), so no kernel is ever launched: the pointers are fake addresses
that are never dereferenced.  The contract follows the page "Check an AI model
calculation before accelerating it", section "The memory contract is part of
the computation" (reject before writing), with the domain of include/rmsnorm.h.
"""
import ctypes
import glob
import os
import re

import pytest

import backward_rmsnorm_fwd_amd as rn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("rmsnorm.h", "layernorm.h",
                                                      "rmsnorm_add.h", "rmsnorm_cast.h")]

pytestmark = pytest.mark.skipif(not os.path.exists(rn.library_path()),
                                reason="librmsnorm.so not built")

OK, ENULL, EDTYPE, ESHAPE, EEPS, EFLAGS, EWS, EALIGN, EOVL = 0, -1, -2, -3, -4, -5, -6, -7, -8
ESTRIDE = -11
A = 0x10000000  # fake, 16-byte aligned "device" addresses; never dereferenced


def lib():
    return rn.load_library()


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+((?:rmsnorm|layernorm)_\w+)\(",
                                 text, re.M)))


def test_every_header_is_scanned():
    assert sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))) == sorted(HEADERS)


def test_header_declares_what_the_binding_knows():
    assert declared_functions() == sorted(rn.EXPORTED_SYMBOLS)


def test_every_declared_symbol_is_exported():
    L = lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings():
    for code in (OK, ENULL, EDTYPE, ESHAPE, EEPS, EFLAGS, EWS, EALIGN, EOVL, -9, -10):
        s = rn.rmsnorm_status_string(code)
        assert s and s != "unknown status"
    assert rn.rmsnorm_status_string(12345) == "unknown status"


def fwd_call(x=A, g=A + (1 << 24), eps=1e-6, M=4, N=256, dtype=2, flags=0,
             y=A + (2 << 24), r=A + (3 << 24)):
    return lib().rmsnorm_fwd(x, g, eps, M, N, dtype, flags, y, r, None)


@pytest.mark.parametrize("kw,code", [
    ({"dtype": 3}, EDTYPE), ({"dtype": -1}, EDTYPE),
    ({"flags": 4}, EFLAGS), ({"flags": 6}, EFLAGS),
    ({"N": 0}, ESHAPE), ({"N": (1 << 24) + 1}, ESHAPE), ({"M": -1}, ESHAPE),
    ({"M": 1 << 40, "N": 65537}, ESHAPE),  # M*N above 2^46
    ({"eps": 0.0}, EEPS), ({"eps": -1e-6}, EEPS), ({"eps": float("nan")}, EEPS),
    ({"eps": float("inf")}, EEPS),
    ({"x": None}, ENULL), ({"g": None}, ENULL), ({"y": None}, ENULL), ({"r": None}, ENULL),
    ({"x": A + 1}, EALIGN), ({"r": A + (3 << 24) + 2}, EALIGN),
    ({"y": A + 8}, EOVL),                # y overlaps x
    ({"r": A + (1 << 24) + 64}, EOVL),   # rstd overlaps gamma
])
def test_fwd_rejects(kw, code):
    assert fwd_call(**kw) == code


def test_fwd_alignment_is_per_element_size():
    # bf16 at a 2-byte boundary is fine for alignment, so the call gets past
    # alignment and is then rejected for the overlap planted with it.
    assert fwd_call(x=A + 2, y=A + 2) == EOVL
    assert fwd_call(x=A + 2, dtype=0) == EALIGN


def test_fwd_m0_is_a_noop_and_needs_no_pointers():
    assert fwd_call(M=0, x=None, g=None, y=None, r=None) == OK


def bwd_call(dy=A, x=A + (1 << 24), g=A + (2 << 24), r=A + (3 << 24), M=4, N=256,
             dtype=2, flags=0, dx=A + (4 << 24), dg=A + (5 << 24), ws=A + (6 << 24),
             ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib().rmsnorm_bwd_workspace_bytes(M, N, dtype, flags)
    return lib().rmsnorm_bwd(dy, x, g, r, M, N, dtype, flags, dx, dg, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    ({"dtype": 5}, EDTYPE), ({"flags": 4}, EFLAGS), ({"N": (1 << 24) + 1}, ESHAPE),
    ({"dy": None}, ENULL), ({"x": None}, ENULL), ({"g": None}, ENULL), ({"r": None}, ENULL),
    ({"dx": None}, ENULL), ({"dg": None}, ENULL),
    ({"ws": None}, EWS), ({"ws_bytes": 16}, EWS),
    ({"ws": A + (6 << 24) + 4}, EALIGN), ({"dy": A + 1}, EALIGN),
    ({"dx": A + 16}, EOVL),               # dx overlaps dy
    ({"dg": A + (3 << 24) + 4}, EOVL),    # dgamma overlaps rstd
    ({"ws": A + (4 << 24) + 256}, EOVL),  # workspace overlaps dx
])
def test_bwd_rejects(kw, code):
    assert bwd_call(**kw) == code


def test_bwd_stage_entry_points_reject():
    L = lib()
    ws = L.rmsnorm_bwd_workspace_bytes(4, 256, 2, 0)
    assert L.rmsnorm_bwd_rows(A, A + (1 << 24), A + (2 << 24), A + (3 << 24), 4, 256, 2, 0,
                              None, A + (6 << 24), ws, None) == ENULL
    assert L.rmsnorm_bwd_rows(A, A + (1 << 24), A + (2 << 24), A + (3 << 24), 4, 256, 2, 0,
                              A + (4 << 24), A + (6 << 24), ws - 4, None) == EWS
    assert L.rmsnorm_bwd_reduce(A, ws, 4, 256, 2, 0, None, None) == ENULL
    assert L.rmsnorm_bwd_reduce(None, ws, 4, 256, 2, 0, A + (5 << 24), None) == EWS
    assert L.rmsnorm_bwd_reduce(A, ws, 4, 256, 2, 0, A + 8, None) == EOVL
    assert L.rmsnorm_bwd_reduce(A, ws, 4, 0, 2, 0, A + (5 << 24), None) == ESHAPE


def test_dgamma_in_dtype_flag():
    """Flag 2 asks for dgamma in the input dtype: accepted by every entry
    point's argument check, same workspace, element-size alignment and span
    for dgamma; unknown bits stay rejected."""
    L = lib()
    ws = L.rmsnorm_bwd_workspace_bytes(4, 256, 2, 0)
    assert L.rmsnorm_bwd_workspace_bytes(4, 256, 2, 2) == ws
    assert L.rmsnorm_bwd_workspace_bytes(4, 256, 2, 3) == ws
    assert L.rmsnorm_bwd_workspace_bytes(4, 256, 2, 4) == 0
    assert L.rmsnorm_bwd_reduce(A, ws, 4, 256, 2, 4, A + (5 << 24), None) == EFLAGS
    # a 2-byte-aligned dgamma is fine for bf16 output, not for float32 output
    assert L.rmsnorm_bwd_reduce(A, ws, 4, 256, 2, 0, A + (5 << 24) + 2, None) == EALIGN
    assert L.rmsnorm_bwd_reduce(A, ws, 4, 256, 2, 2, A + (5 << 24) + 1, None) == EALIGN
    # the bf16 dgamma span is N*2 = 512 bytes: starting 2 bytes in, it
    # reaches 2 bytes into a workspace placed 512 bytes after its base
    assert L.rmsnorm_bwd_reduce(A + 512, ws, 4, 256, 2, 2, A + 2, None) == EOVL


def fwd_strided_call(x=A, ldx=256, g=A + (1 << 24), eps=1e-6, M=4, N=256, dtype=2, flags=0,
                     y=A + (2 << 24), ldy=256, r=A + (3 << 24)):
    return lib().rmsnorm_fwd_strided(x, ldx, g, eps, M, N, dtype, flags, y, ldy, r, None)


@pytest.mark.parametrize("kw,code", [
    ({"ldx": 255}, ESTRIDE), ({"ldy": 0}, ESTRIDE), ({"ldx": -256}, ESTRIDE),
    ({"ldx": (1 << 40) + 1}, ESTRIDE), ({"flags": 4}, EFLAGS), ({"y": None}, ENULL),
    # y starts half a row into x's rows at the same stride: they share bytes
    ({"ldx": 512, "ldy": 512, "y": A + 256}, EOVL),
    # y one element before the end of x's first row, at x's stride
    ({"ldx": 512, "ldy": 512, "y": A + 510}, EOVL),
    # different strides with overlapping extents count as overlapping
    ({"ldx": 512, "ldy": 768, "y": A + 512}, EOVL),
    # the weight inside the gaps of strided x is still an input: y may not hit it
    ({"ldx": 512, "ldy": 256, "g": A + 512, "y": A + 512 + 128}, EOVL),
])
def test_fwd_strided_rejects(kw, code):
    assert fwd_strided_call(**kw) == code


def test_bwd_strided_rejects():
    L = lib()
    ws = L.rmsnorm_bwd_workspace_bytes(4, 256, 2, 0)
    args = dict(dy=A, lddy=256, x=A + (1 << 24), ldx=256, g=A + (2 << 24), r=A + (3 << 24),
                dx=A + (4 << 24), lddx=256, dg=A + (5 << 24), ws=A + (6 << 24))

    def call(**kw):
        a = dict(args, **kw)
        return L.rmsnorm_bwd_strided(a["dy"], a["lddy"], a["x"], a["ldx"], a["g"], a["r"], 4,
                                     256, 2, 0, a["dx"], a["lddx"], a["dg"], a["ws"], ws, None)
    assert call(lddy=100) == ESTRIDE and call(ldx=255) == ESTRIDE and call(lddx=1) == ESTRIDE
    # dx interleaved half a row into dy's rows (same stride 512): overlap
    assert call(lddy=512, lddx=512, dx=A + 256) == EOVL
    assert call(dg=None) == ENULL


# Layouts whose span (M - 1) * pitch passes 2^63 (or the 2^57 address limit)
# with y == x: validation must refuse them (a stride error), never let them
# reach a launch.  Before spans were formed in 128 bits, (M - 1) * pitch
# wrapped and M = 2^40, ld = 2^40 passed validation.
@pytest.mark.parametrize("ld", [1 << 40, 1 << 22, 1 << 30])
@pytest.mark.parametrize("dtype", [0, 1, 2])
def test_fwd_strided_span_past_the_address_limit(ld, dtype):
    M = 1 << 40
    assert fwd_strided_call(x=A, ldx=ld, y=A, ldy=ld, M=M, N=1, dtype=dtype) == ESTRIDE
    assert fwd_strided_call(x=A, ldx=ld, M=M, N=1, dtype=dtype) == ESTRIDE


def test_bwd_strided_span_past_the_address_limit():
    L = lib()
    for ld in (1 << 40, 1 << 22):
        st = L.rmsnorm_bwd_strided(A, ld, A, ld, A + 64, A + 128, 1 << 40, 1, 2, 0, A, ld,
                                   A + 256, A + 512, 1 << 40, None)
        assert st == ESTRIDE


def test_dense_rows_past_the_address_limit():
    top = (1 << 57) - 1024
    assert fwd_call(x=top) == ESHAPE


def test_overlap_found_at_large_pitches():
    # y's row 0 is x's row 1 with a pitch of 2^40 elements (2^41 bytes):
    # the extent (about 2^55 bytes) fits, the rows meet.
    ld = 1 << 40
    assert fwd_strided_call(x=A, ldx=ld, y=A + 2 * ld, ldy=ld, M=1 << 14, N=8) == EOVL


def test_bwd_noalloc_rejects():
    """The allocation-free backward checks every caller argument, and the need
    against its fixed buffer, before it looks the buffer up on a device."""
    L = lib()
    S = 1 << 24

    def call(dy=A, x=A + S, g=A + 2 * S, r=A + 3 * S, M=4, N=256, dtype=2, flags=0,
             dx=A + 4 * S, dg=A + 5 * S):
        return L.rmsnorm_bwd_noalloc(dy, x, g, r, M, N, dtype, flags, dx, dg, None)
    # 32 rows of 2^24 float32 need two 64 MiB partial rows + the split
    # plan's row sums: too big
    assert L.rmsnorm_bwd_workspace_bytes(32, 1 << 24, 0, 0) > rn.NOALLOC_SCRATCH_BYTES
    big = 32 << 26
    assert call(dy=A, x=A + big, g=A + 2 * big, r=A + 3 * big, M=32, N=1 << 24, dtype=0,
                dx=A + 4 * big, dg=A + 5 * big) == EWS
    assert call(dtype=5) == EDTYPE and call(flags=8) == EFLAGS and call(N=0) == ESHAPE
    assert call(dy=None) == ENULL and call(dg=None) == ENULL and call(r=None) == ENULL
    assert call(x=A + S + 1) == EALIGN and call(dg=A + 5 * S + 2) == EALIGN
    assert call(dx=A + S + 64) == EOVL        # dx overlaps x
    assert call(dg=A + 2 * S + 4) == EOVL     # dgamma overlaps gamma
    assert call(dg=A + 4 * S + 8) == EOVL     # dgamma overlaps dx
    assert "RMSNORM_NOALLOC_SCRATCH_BYTES" in rn.rmsnorm_status_string(EWS)


def test_shape_status_string_names_each_family_limit():
    s = rn.rmsnorm_status_string(-3)
    assert "2^24" in s and "2^46" in s and "layernorm_" in s and "rmsnorm_cast_" in s


def test_stride_status_string():
    assert "stride" in rn.rmsnorm_status_string(ESTRIDE)


def test_workspace_bytes():
    L = lib()
    assert L.rmsnorm_bwd_workspace_bytes(0, 4096, 2, 0) == 0
    assert L.rmsnorm_bwd_workspace_bytes(4, 0, 2, 0) == 0      # invalid -> 0
    assert L.rmsnorm_bwd_workspace_bytes(4, 4096, 9, 0) == 0   # invalid -> 0
    r4 = lambda v: -(-v // 4) * 4  # noqa: E731
    for (m, n, dt) in [(32768, 4096, 2), (262144, 1024, 1), (2048, 65536, 2),
                       (65536, 5120, 2), (65, 128, 0), (1, 2, 0), (16, 16384, 0),
                       (2048, 65535, 2), (4096, 20000, 0)]:
        p = rn.rmsnorm_query_plan(m, n, dt, which=rn.PASS_BWD_ROWS)
        ws = L.rmsnorm_bwd_workspace_bytes(m, n, dt, 0)
        if n <= 16384:
            assert ws == p["partials"] * n * 4
        else:
            # past 16384 any layout may run the split kernels, so the
            # workspace also holds their per-(row, segment) sums and
            # per-row coefficients
            nseg = -(-n * (4 if dt == 0 else 2) // 16384)
            assert ws == 4 * (r4(p["partials"] * n) + r4(m * nseg) + r4(m))
        assert 1 <= p["partials"] <= m
        # the workspace is far below the page's M x N float32 partial array
        assert ws <= m * n * 4


def test_plans_for_the_workloads():
    """The full-width kernels serve the five workloads (aligned pointers)."""
    c2 = rn.rmsnorm_query_plan(32768, 4096, 2, which=rn.PASS_FWD)
    assert c2["kernel_name"] == "fwd_pipe" and c2["vec"] == 8 and c2["x_in_lds"] == 1
    assert (c2["threads_per_row"], c2["chunks"], c2["block_threads"]) == (256, 2, 1024)
    assert c2["grid"] == 512 and c2["lds_bytes"] == 2 * 4 * 4096 * 2
    b2 = rn.rmsnorm_query_plan(32768, 4096, 2, which=rn.PASS_BWD_ROWS)
    assert b2["kernel_name"] == "bwd_rows" and b2["x_in_lds"] == 1
    assert (b2["threads_per_row"], b2["chunks"], b2["partials"]) == (256, 2, 512)
    assert b2["block_threads"] == 512 and b2["lds_bytes"] == 2 * 4096 * 2
    b3 = rn.rmsnorm_query_plan(262144, 1024, 1, which=rn.PASS_BWD_ROWS)
    assert b3["kernel_name"] == "bwd_pipe" and b3["dy_in_lds"] == 0
    assert (b3["threads_per_row"], b3["chunks"], b3["partials"]) == (128, 1, 256)
    assert b3["lds_bytes"] == 2 * 8 * 1024 * 2
    c3 = rn.rmsnorm_query_plan(262144, 1024, 1, which=rn.PASS_FWD)
    assert c3["kernel_name"] == "fwd_rows" and (c3["threads_per_row"], c3["chunks"]) == (64, 2)
    c4 = rn.rmsnorm_query_plan(2048, 65536, 2, which=rn.PASS_BWD_ROWS)
    assert c4["kernel_name"] == "bwd_long" and c4["threads_per_row"] == 512
    assert c4["chunks"] == 16 and c4["partials"] == 256
    assert c4["x_in_lds"] == 1 and c4["lds_bytes"] == 65536 * 2
    c5 = rn.rmsnorm_query_plan(65536, 5120, 2, offset=True, which=rn.PASS_BWD_ROWS)
    assert c5["kernel_name"] == "bwd_pipe" and (c5["threads_per_row"], c5["chunks"]) == (640, 1)
    assert c5["block_threads"] == 640
    assert c5["dy_in_lds"] == 1 and c5["partials"] == 256 and c5["lds_bytes"] == 2 * 2 * 5120 * 2
    f5 = rn.rmsnorm_query_plan(65536, 5120, 2, offset=True, which=rn.PASS_FWD)
    assert f5["kernel_name"] == "fwd_rows" and (f5["threads_per_row"], f5["chunks"]) == (320, 2)
    assert f5["block_threads"] == 640
    # odd N forces element-wide accesses; misaligned pointers narrow the vector
    odd = rn.rmsnorm_query_plan(3, 257, 2, which=rn.PASS_FWD)
    assert odd["vec"] == 1 and odd["kernel_name"] == "fwd_wave"
    mis = rn.rmsnorm_query_plan(8, 4096, 2, which=rn.PASS_FWD, align_bytes=4)
    assert mis["vec"] == 2 and mis["kernel_name"] in ("fwd_wave", "fwd_block")
    red = rn.rmsnorm_query_plan(32768, 4096, 2, which=rn.PASS_BWD_REDUCE)
    assert red["kernel_name"] == "bwd_reduce16" and red["grid"] == 4096 // 16
    red4 = rn.rmsnorm_query_plan(2048, 65536, 2, which=rn.PASS_BWD_REDUCE)
    assert red4["kernel_name"] == "bwd_reduce_wide" and red4["grid"] == 65536 // 256
    assert red4["block_threads"] == 1024


def test_partials_do_not_depend_on_alignment():
    for (m, n, dt) in [(32768, 4096, 2), (999, 5120, 2), (5, 4104, 2), (7, 2048, 0)]:
        ps = {rn.rmsnorm_query_plan(m, n, dt, which=rn.PASS_BWD_ROWS, align_bytes=a)["partials"]
              for a in (16, 8, 4)}
        assert len(ps) == 1, (m, n, dt, ps)


def test_full_width_plan_used_for_aligned_rows():
    """Every N whose rows are 16-byte multiples gets a listed full-width
    kernel, except float32 rows beyond 32768 in the backward (split rows)."""
    for dt, es in ((0, 4), (1, 2), (2, 2)):
        vec = 16 // es
        for n in range(vec, 65537, vec * 7):
            f = rn.rmsnorm_query_plan(5, n, dt, which=rn.PASS_FWD)
            assert f["kernel_name"] in ("fwd_rows", "fwd_pipe"), (dt, n)
            assert (f["kernel_name"] == "fwd_pipe") == (4096 < n * es <= 8192), (dt, n)
            b = rn.rmsnorm_query_plan(5, n, dt, which=rn.PASS_BWD_ROWS)
            if dt == 0 and n > 32768:
                assert b["kernel_name"] == "bwd_split", (dt, n)
            else:
                assert b["kernel_name"] in ("bwd_rows", "bwd_pipe", "bwd_long"), (dt, n)
                pipe = n * es <= 4096 or 8192 < n * es <= 16384
                assert (b["kernel_name"] == "bwd_pipe") == pipe, (dt, n)
                assert (b["kernel_name"] == "bwd_long") == (n * es > 16384), (dt, n)


def test_plan_covers_every_n():
    """Every N in the domain gets a plan whose threads cover the row."""
    for dt in (0, 1, 2):
        for n in list(range(1, 300)) + [1023, 1024, 1025, 4095, 4096, 4097, 5120, 8191,
                                         8192, 8193, 16383, 16385, 32767, 32769,
                                         65535, 65536]:
            for which in (rn.PASS_FWD, rn.PASS_BWD_ROWS):
                for align in (16, 8, 4, 2):
                    if dt == 0 and align < 4:
                        continue
                    p = rn.rmsnorm_query_plan(7, n, dt, which=which, align_bytes=align)
                    assert n % p["vec"] == 0
                    if p["kernel_name"].endswith("_split"):
                        # rows over 16384 that no full-width kernel takes
                        seg = 256 * p["chunks"] * p["vec"]
                        assert n > 16384 and p["segments"] * seg >= n > (p["segments"] - 1) * seg
                        continue
                    assert p["threads_per_row"] * p["chunks"] * p["vec"] >= n
                    assert p["threads_per_row"] * (p["chunks"] - 1) * p["vec"] < n
                    assert p["chunks"] <= 64 and p["block_threads"] <= 1024
                    assert p["lds_bytes"] <= 160 * 1024


def _ceil(a, b):
    return -(-a // b)


@pytest.mark.parametrize("M,N,dt", [(33, 131072, 2), (5, 65537, 1), (7, 65540, 0),
                                    (2, 1 << 24, 2), (261, 98304, 2), (100000, 70000, 1),
                                    (1, 1 << 24, 0), (4096, 65537, 0)])
def test_split_plan(M, N, dt):
    """Rows longer than 65536 elements: 16 KiB segments, one 256-thread
    workgroup per (row block, segment), blocks of at least 16 rows where M
    allows; the workspace holds the [P, N] column partials, the [M, segments]
    row partials and the [M] coefficients, each from a 16-byte boundary."""
    es = 4 if dt == 0 else 2
    nseg = _ceil(N * es, 16384)
    f = rn.rmsnorm_query_plan(M, N, dt, which=rn.PASS_FWD)
    b = rn.rmsnorm_query_plan(M, N, dt, which=rn.PASS_BWD_ROWS)
    assert f["kernel_name"] == "fwd_split" and b["kernel_name"] == "bwd_split"
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
    # the forward keeps no column sums: one row per block
    assert f["grid"] // nseg == max(1, min(M, ((1 << 24) - 1) // nseg))
    r4 = lambda v: _ceil(v, 4) * 4  # noqa: E731
    assert rn.rmsnorm_bwd_workspace_bytes(M, N, dt) == 4 * (r4(P * N) + r4(M * nseg) + r4(M))
    red = rn.rmsnorm_query_plan(M, N, dt, which=rn.PASS_BWD_REDUCE)
    assert red["partials"] == P
    if N % 4 == 0:
        assert red["kernel_name"] == "bwd_reduce_wide" and red["grid"] == _ceil(N, 256)
        slices = 1
        while slices < min(16, _ceil(P, 4)):
            slices *= 2
        assert red["block_threads"] == 64 * slices
    else:
        assert red["kernel_name"] == "bwd_reduce"


def test_split_plan_covers_rows_and_scratch():
    """Every split N: the segments cover the row with no empty segment, and a
    row of y has room for the forward's per-segment float32 sums (two 16-bit
    or one 32-bit element each)."""
    for dt in (0, 1, 2):
        es = 4 if dt == 0 else 2
        for n in [65537, 65540, 65544, 73728, 98303, 131072, 131073, 999999, (1 << 24) - 1,
                  1 << 24]:
            for align in (16, 8, 4, 2):
                if es == 4 and align < 4:
                    continue
                p = rn.rmsnorm_query_plan(3, n, dt, which=rn.PASS_FWD, align_bytes=align)
                seg = 256 * p["chunks"] * p["vec"]
                assert seg * es == 16384 and n % p["vec"] == 0
                assert p["segments"] * seg >= n > (p["segments"] - 1) * seg
                assert p["segments"] * (4 // es) <= n
    assert rn.rmsnorm_query_plan(3, 65536, 2, which=rn.PASS_FWD)["kernel_name"] != "fwd_split"
    # rows over 16384 that no full-width kernel takes run the split kernels
    # too: odd N, narrow alignment, float32 backward rows over 128 KiB
    for (n, dt, align, which) in [(65535, 2, 16, rn.PASS_FWD), (20001, 1, 16, rn.PASS_BWD_ROWS),
                                  (40000, 2, 4, rn.PASS_FWD), (65536, 0, 16, rn.PASS_BWD_ROWS),
                                  (40000, 0, 16, rn.PASS_BWD_ROWS)]:
        p = rn.rmsnorm_query_plan(3, n, dt, which=which, align_bytes=align)
        assert p["kernel_name"].endswith("_split"), (n, dt, align)
    for (n, dt, align) in [(16383, 2, 16), (16384, 0, 4), (4097, 1, 16)]:
        p = rn.rmsnorm_query_plan(3, n, dt, which=rn.PASS_BWD_ROWS, align_bytes=align)
        assert p["kernel_name"] in ("bwd_wave", "bwd_block"), (n, dt, align)
    with pytest.raises(rn.RmsnormError):
        rn.rmsnorm_query_plan(3, (1 << 24) + 1, 2)


def test_query_plan_rejects():
    L = lib()
    p = rn.Plan()
    assert L.rmsnorm_query_plan(4, 256, 2, 0, 7, 16, ctypes.byref(p)) == -10
    assert L.rmsnorm_query_plan(4, 256, 2, 0, 0, 3, ctypes.byref(p)) == -10
    assert L.rmsnorm_query_plan(4, 256, 2, 0, 0, 16, None) == ENULL
