"""The explicit memory waits of the pipelined backward kernels, checked on
their compiled gfx950 assembly (no GPU needed).

Those kernels prefetch dy with loads the compiler does not track, so the
compiler neither waits for them nor keeps their registers from other values
while they are in flight; only the kernel's own `s_waitcnt vmcnt(k)` and
the asm operands do.  Any compiler change could undo that, so every build
is checked here: the full-width instantiations of each dtype are compiled
to assembly and every untracked load is followed along every path until a
wait completes it (tests/asm_waits.py).  The checker itself is pinned on
small hand-written listings and on mutants of the real code: any one
explicit wait dropped or made one count weaker, or a register of a load in
flight read, must be reported."""
import os
import re
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

import asm_waits
from backward_rmsnorm_fwd_amd import build

DTYPES = ("kF32", "kF16", "kBF16")


@pytest.fixture(scope="module")
def listings():
    """{dtype: assembly of the full-width instantiations}."""
    with tempfile.TemporaryDirectory(prefix="rmsnorm_asm_") as tmp:
        def compile_one(dt):
            out = os.path.join(tmp, f"inst_{dt}.s")
            cmd = [build.hipcc(), *build.FLAGS, "-I", os.path.join(build.ROOT, "include"),
                   f"-DRMSNORM_INST_DT={dt}", "--offload-device-only", "-S",
                   os.path.join(build.CSRC, "rmsnorm_fast_inst.hip"), "-o", out]
            res = subprocess.run(cmd, capture_output=True, text=True)
            assert res.returncode == 0, res.stderr[-2000:]
            with open(out) as f:
                return dt, f.read()

        with ThreadPoolExecutor(len(DTYPES)) as ex:
            return dict(ex.map(compile_one, DTYPES))


def _pipe(name):
    return "bwd_pipe_kernel" in name


def _count(lines):
    return len(asm_waits.check_function(lines)[0])


@pytest.mark.parametrize("dt", DTYPES)
def test_untracked_loads_complete_before_use(listings, dt):
    res = asm_waits.check_listing(listings[dt])
    # only the pipelined backward holds untracked loads: the register-dy
    # variants with one, two and four wavefronts per row
    assert res and all(_pipe(name) for name in res), sorted(res)
    assert len(res) == 3, sorted(res)
    for name, (violations, n) in res.items():
        assert n >= 2, name
        assert not violations, (name, violations[:5])


@pytest.mark.parametrize("dt", DTYPES)
def test_checker_reports_mutants_of_the_real_code(listings, dt):
    fns = asm_waits.functions(listings[dt])
    checked = 0
    for name, lines in fns.items():
        if not _pipe(name) or not asm_waits.check_listing(listings[dt], lambda n: n == name):
            continue
        waits = asm_waits.explicit_waits(lines)
        assert len(waits) >= 6, name  # two choices in each step of the unrolled loop
        for i in waits:
            assert _count(lines[:i] + lines[i + 1:]), ("dropped", name, i)
            k = int(asm_waits._VMCNT.search(lines[i][0]).group(1))
            weaker = list(lines)
            weaker[i] = (f"s_waitcnt vmcnt({k + 1})", True)
            assert _count(weaker), ("weakened", name, i)
        for i, (text, in_asm) in enumerate(lines):
            m = asm_waits._UNTRACKED.match(text) if in_asm else None
            if m:
                early = list(lines)
                early.insert(i + 1, (f"v_mov_b32 v255, v{m.group(2)}", False))
                assert _count(early), ("early read", name, i)
        checked += 1
    assert checked == 3


def _listing(body):
    """A one-function listing from instruction lines; lines starting with
    '@' are inside an inline-asm block."""
    out = ["_Z1fv:"]
    for line in body.strip().splitlines():
        line = line.strip()
        if line.startswith("@"):
            out += [";;#ASMSTART", "\t" + line[1:].strip(), ";;#ASMEND"]
        else:
            out.append(line if line.endswith(":") else "\t" + line)
    out.append(".Lfunc_end0:")
    return "\n".join(out) + "\n"


def _violations(body):
    res = asm_waits.check_listing(_listing(body))
    return res["_Z1fv"][0] if res else None


LOAD = "@global_load_dwordx4 v[4:7], v[0:1], off nt"
STORE = "global_store_dwordx4 v[8:9], v[10:13], off"


def test_checker_on_straight_line_code():
    assert _violations(f"{LOAD}\n@s_waitcnt vmcnt(0)\nv_add_f32 v2, v4, v5\ns_endpgm") == []
    assert _violations(f"{LOAD}\nv_add_f32 v2, v4, v5\n@s_waitcnt vmcnt(0)\ns_endpgm")
    # one store after the load: vmcnt(1) completes the load, vmcnt(2) does not
    assert _violations(f"{LOAD}\n{STORE}\n@s_waitcnt vmcnt(1)\nv_mov_b32 v2, v7\ns_endpgm") == []
    assert _violations(f"{LOAD}\n{STORE}\n@s_waitcnt vmcnt(2)\nv_mov_b32 v2, v7\ns_endpgm")
    # a register of the load written by another instruction while in flight
    assert _violations(f"{LOAD}\nv_mov_b32 v6, 0\n@s_waitcnt vmcnt(0)\ns_endpgm")
    # the load's own address registers may overlap its destination
    assert _violations("@global_load_dwordx4 v[4:7], v[4:5], off nt\n"
                       "@s_waitcnt vmcnt(0)\nv_mov_b32 v2, v4\ns_endpgm") == []


def test_checker_follows_branches_and_loops():
    # a use reached by a branch that skips the wait
    assert _violations(f"""
        {LOAD}
        s_cbranch_scc1 .LBB0_2
        @s_waitcnt vmcnt(0)
        v_mov_b32 v3, 0
        .LBB0_2:
        v_mov_b32 v2, v4
        s_endpgm""")
    # ...but a branch over nothing but the waits is the inactive row, for
    # which no prefetch was issued (the checker's stated assumption)
    assert _violations(f"""
        {LOAD}
        s_cbranch_scc1 .LBB0_2
        @s_waitcnt vmcnt(0)
        .LBB0_2:
        v_mov_b32 v2, v4
        s_endpgm""") == []
    # a loop whose next pass reads the load issued by the previous one
    assert _violations(f"""
        .LBB0_1:
        v_mov_b32 v2, v4
        {LOAD}
        s_cbranch_scc1 .LBB0_1
        @s_waitcnt vmcnt(0)
        s_endpgm""")
    assert _violations(f"""
        .LBB0_1:
        @s_waitcnt vmcnt(0)
        v_mov_b32 v2, v4
        {LOAD}
        s_cbranch_scc1 .LBB0_1
        @s_waitcnt vmcnt(0)
        s_endpgm""") == []


def test_checker_wait_choice_regions():
    # inactive row skips both waits; the two choices are made on one mask
    region = """
        s_cbranch_vccnz .LBB0_3
        s_mov_b64 s[0:1], -1
        s_and_b64 vcc, exec, s[4:5]
        s_cbranch_vccz .LBB0_2
        @s_waitcnt vmcnt({a})
        s_mov_b64 s[0:1], 0
        .LBB0_2:
        s_andn2_b64 vcc, exec, s[0:1]
        s_cbranch_vccnz .LBB0_3
        @s_waitcnt vmcnt({b})
        .LBB0_3:"""
    lines = asm_waits.functions(_listing(region.format(a=0, b=1)))["_Z1fv"]
    assert [w for _, _, w in asm_waits._wait_regions(lines)] == [[1, 0]]
    # one store after the load when its lane reaches the last chunk, none
    # otherwise: waits 1 and 0 are exact, either one count weaker is not
    body = """
        {load}
        s_and_saveexec_b64 s[2:3], s[6:7]
        s_cbranch_execz .LBB0_1
        {store}
        .LBB0_1:
        s_or_b64 exec, exec, s[2:3]
        {region}
        v_mov_b32 v2, v4
        s_endpgm"""
    for a, b, bad in ((0, 1, False), (1, 1, True), (0, 2, True)):
        v = _violations(body.format(load=LOAD, store=STORE, region=region.format(a=a, b=b)))
        assert bool(v) == bad, (a, b)
    # a region that leaves one choice without a wait
    v = _violations(body.format(load=LOAD, store=STORE, region=region.format(a=0, b=1).replace(
        "@s_waitcnt vmcnt(1)", "s_nop 0")))
    assert v


def test_regions_found_on_the_real_code_choose_store_counts(listings):
    """Each step waits with one of two counts that differ by one: the stores
    of the previous row with and without the last chunk's."""
    for dt in DTYPES:
        for name, lines in asm_waits.functions(listings[dt]).items():
            if not _pipe(name):
                continue
            for _, _, waits in asm_waits._wait_regions(lines):
                assert None not in waits and len(set(waits)) == 2, (name, waits)
                assert max(waits) - min(waits) == 1, (name, waits)
