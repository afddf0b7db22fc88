"""Static check of the explicit memory waits in compiled gfx950 assembly.

The pipelined backward kernels prefetch dy into registers with loads written
in inline asm, which the compiler does not track: nothing but the kernel's
own `s_waitcnt vmcnt(k)` guarantees such a load has landed before its
registers are read, and nothing but the asm operands that tie the
registers keeps the compiler from giving them to other values while the
load is in flight.  This module checks both on the compiled code.

gfx9 counts vector-memory operations (loads, stores, LDS DMA) on one
in-order counter: after `s_waitcnt vmcnt(k)` at most the k most recent ones
are outstanding.  A load is therefore complete at such a wait once at least
k vector-memory operations were issued after it.  The check follows every
path of each function's control-flow graph, tracking for every untracked
load in flight how many vector-memory operations were issued after it, and
reports any instruction other than the load itself that names one of the
load's destination registers while the load may still be in flight.

The kernels choose at run time whether and how long to wait, on facts a
path-insensitive analysis cannot see; the check takes them as follows.
  * A wait region is a run of scalar instructions, conditional branches
    and waits.  Its scalar masks are taken as unknown uniform booleans and
    every combination is run, which yields the count each feasible path
    waits with (or shows a path that does not wait).
  * A branch over nothing but a region's waits is the inactive row: the
    kernels issue a row's prefetch under the same condition, so nothing is
    in flight there.
  * The counts are chosen by whether the wavefront's lanes reach the last
    chunk, the same fact that decides whether the last chunk's store runs.
    Two executions are checked: every store runs and each region waits with
    its weakest count; or the stores that a branch on the execution mask
    skips are skipped and each region waits with its strongest count.
"""
import re

_FUNC = re.compile(r"^(_Z\S+):", re.M)
_LABEL = re.compile(r"^(\.L\w+):")
_BRANCH = re.compile(r"^\s*(s_cbranch_\w+|s_branch)\s+(\.L\w+)")
_VMCNT = re.compile(r"\bvmcnt\((\d+)\)")
_VREG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")
_UNTRACKED = re.compile(r"^\s*global_load_dword\w*\s+v\[(\d+):(\d+)\],.*\boff\b")
_VMEM = re.compile(r"^\s*(global_|buffer_|flat_|scratch_)")
_SOP = re.compile(r"^\s*(s_(?:mov|and|andn2|or|xor|not)_b64)\s+(vcc|s\[\d+:\d+\]),\s*(.+)$")
_CAP = 64  # larger than any wait count the kernels use


def functions(asm):
    """{mangled name: list of instruction lines, asm-block flag} for each
    function of an assembly listing."""
    out = {}
    starts = [(m.group(1), m.end()) for m in _FUNC.finditer(asm)]
    for name, pos in starts:
        end = asm.find(".Lfunc_end", pos)
        body = asm[pos:end if end >= 0 else len(asm)]
        lines, in_asm = [], False
        for raw in body.splitlines():
            text = raw.split(";", 1)[0].rstrip() if ";;#" not in raw else raw.strip()
            if text == ";;#ASMSTART":
                in_asm = True
                continue
            if text == ";;#ASMEND":
                in_asm = False
                continue
            if text.strip():
                lines.append((text, in_asm))
        out[name] = lines
    return out


def _regs(text):
    """VGPR numbers an instruction names (its operands)."""
    parts = text.split(None, 1)
    if len(parts) < 2:
        return set()
    regs = set()
    for m in _VREG.finditer(parts[1]):
        if m.group(3) is not None:
            regs.add(int(m.group(3)))
        else:
            regs.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return regs


def _blocks(lines):
    """Basic blocks: list of (label or None, instructions, successor labels)."""
    blocks, cur_label, cur = [], None, []

    def close(succ):
        blocks.append([cur_label, cur, succ])

    for text, in_asm in lines:
        m = _LABEL.match(text)
        if m:
            if cur or cur_label is not None:
                close(["<next>"])
            cur_label, cur = m.group(1), []
            continue
        cur.append((text, in_asm))
        b = _BRANCH.match(text)
        if b:
            succ = [b.group(2)] + (["<next>"] if b.group(1).startswith("s_cbranch") else [])
            close(succ)
            cur_label, cur = None, []
        elif text.strip().startswith("s_endpgm"):
            close([])
            cur_label, cur = None, []
    if cur:
        close(["<next>"])
    index = {b[0]: i for i, b in enumerate(blocks) if b[0] is not None}
    resolved = []
    for i, (label, insts, succ) in enumerate(blocks):
        nxt = []
        for s in succ:
            if s == "<next>":
                if i + 1 < len(blocks):
                    nxt.append(i + 1)
            elif s in index:
                nxt.append(index[s])
        resolved.append((label, insts, nxt))
    return resolved


def _wait_regions(lines):
    """Regions of explicit waits chosen at run time: [(first, last, path
    waits)], where path waits holds, for each path through the region that
    must wait, the strongest count it waits with (None for a path with no
    wait at all).

    A region is a run of scalar instructions, conditional branches, labels
    and waits whose branches all land further on inside it, at its end, or
    on one-instruction trampolines back into it, and whose inner labels are
    reached from nowhere else.  The pipelined kernels wait for a row's
    prefetch only when the row is active (a prefetch was issued for it
    exactly then), so the region's first branch, when it jumps to the end,
    is the inactive row and needs no wait; every other path must wait."""
    n = len(lines)
    label_at, sources = {}, {}
    for i, (t, _) in enumerate(lines):
        m = _LABEL.match(t)
        if m:
            label_at[m.group(1)] = i
        b = _BRANCH.match(t)
        if b:
            sources.setdefault(b.group(2), []).append(i)
    tramp = {}  # trampoline label -> (index of its branch, destination)
    for lab, i in label_at.items():
        if i + 1 < n:
            b = _BRANCH.match(lines[i + 1][0])
            if b and b.group(1) == "s_branch":
                tramp[lab] = (i + 1, b.group(2))

    def extent(i):
        j, targets, labels, tramps = i, set(), set(), set()
        while j < n:
            t = lines[j][0].strip()
            bb = _BRANCH.match(t)
            lab = _LABEL.match(t)
            if bb and bb.group(1).startswith("s_cbranch"):
                dest = bb.group(2)
                if dest in tramp:
                    tramps.add(dest)
                    dest = tramp[dest][1]
                targets.add(dest)
            elif lab:
                labels.add(lab.group(1))
                if targets <= labels:
                    return j, labels, tramps
            elif not t.startswith("s_") or t.startswith(("s_branch", "s_endpgm", "s_barrier")):
                return None
            j += 1
        return None

    def runs(p, j):
        """Strongest wait of each run from line p to the region's end j, the
        region's scalar masks taken as unknown uniform booleans (every
        combination is run), or None when the region computes its branch
        conditions in a way this does not model."""
        code, atoms = [], []
        for q in range(p, j):
            t = lines[q][0].strip()
            if _LABEL.match(t):
                code.append(("label", _LABEL.match(t).group(1)))
                continue
            w = _VMCNT.search(t) if t.startswith("s_waitcnt") else None
            if w:
                code.append(("wait", int(w.group(1))))
                continue
            if t.startswith("s_waitcnt"):
                continue
            bb = _BRANCH.match(t)
            if bb:
                dest = tramp[bb.group(2)][1] if bb.group(2) in tramp else bb.group(2)
                code.append(("br", bb.group(1), dest))
                continue
            m = _SOP.match(t)
            if not m:
                return None
            op, dst, srcs = m.group(1), m.group(2), [x.strip() for x in m.group(3).split(",")]
            for x in srcs:
                if x not in ("exec", "0", "-1") and x not in atoms and \
                        not any(c[0] == "op" and c[2] == x for c in code):
                    atoms.append(x)
            code.append(("op", op, dst, srcs))
        if len(atoms) > 6:
            return None
        at = {c[1]: k for k, c in enumerate(code) if c[0] == "label"}
        results = []
        for bits in range(1 << len(atoms)):
            env = {x: bool(bits >> k & 1) for k, x in enumerate(atoms)}
            val = lambda x: True if x in ("exec", "-1") else False if x == "0" else env[x]
            k, strongest = 0, None
            while k < len(code):
                c = code[k]
                if c[0] == "wait":
                    strongest = c[1] if strongest is None else min(strongest, c[1])
                elif c[0] == "op":
                    v = [val(x) for x in c[3]]
                    env[c[2]] = {"s_mov_b64": lambda: v[0], "s_and_b64": lambda: v[0] and v[1],
                                 "s_andn2_b64": lambda: v[0] and not v[1],
                                 "s_or_b64": lambda: v[0] or v[1],
                                 "s_xor_b64": lambda: v[0] != v[1],
                                 "s_not_b64": lambda: not v[0]}[c[1]]()
                elif c[0] == "br":
                    cond = {"s_cbranch_vccnz": lambda: env["vcc"], "s_cbranch_vccz":
                            lambda: not env["vcc"], "s_cbranch_execnz": lambda: True,
                            "s_cbranch_execz": lambda: False}.get(c[1])
                    if cond is None:
                        return None
                    if cond():
                        if c[2] not in at:
                            break  # the region's end
                        k = at[c[2]]
                        continue
                k += 1
            results.append(strongest)
        return results

    def paths(p, j, strongest):
        """Strongest wait on each path from line p to the region's end j."""
        while p < j:
            t = lines[p][0].strip()
            bb = _BRANCH.match(t)
            if bb and bb.group(1).startswith("s_cbranch"):
                dest = bb.group(2)
                dest = tramp[dest][1] if dest in tramp else dest
                q = label_at.get(dest, -1)
                if not p < q <= j:
                    raise ValueError("branch leaves the wait region")
                return paths(q, j, strongest) + paths(p + 1, j, strongest)
            w = _VMCNT.search(t) if t.startswith("s_waitcnt") else None
            if w:
                k = int(w.group(1))
                strongest = k if strongest is None else min(strongest, k)
            p += 1
        return [strongest]

    out, i = [], 0
    while i < n:
        b = _BRANCH.match(lines[i][0])
        r = extent(i) if b and b.group(1).startswith("s_cbranch") else None
        if r:
            j, labels, tramps = r
            end = _LABEL.match(lines[j][0]).group(1)
            tramp_src = {tramp[t][0] for t in tramps}
            inner_ok = all(i <= src <= j or src in tramp_src
                           for lab in (labels - {end}) | tramps for src in sources.get(lab, []))
            inner_ok = inner_ok and all(i <= src <= j for t in tramps for src in sources.get(t, []))
            has_wait = any(_VMCNT.search(lines[q][0]) for q in range(i, j))
            if inner_ok and has_wait:
                first = _BRANCH.match(lines[i][0]).group(2)
                first = tramp[first][1] if first in tramp else first
                p = i + 1 if first == end else i
                waits = runs(p, j)
                if waits is None:
                    waits = paths(p, j, None)
                out.append((i, j, waits))
                i = j + 1
                continue
        i += 1
    return out


def _collapse(lines, regions, pick):
    """The listing with each wait region replaced by the wait `pick` chooses
    from its paths' waits (none at all when a path does not wait)."""
    out, pos = [], 0
    for i, j, waits in regions:
        out.extend(lines[pos:i])
        if None not in waits:
            out.append((f"s_waitcnt vmcnt({pick(waits)})", True))
        out.extend(l for l in lines[i:j + 1] if _LABEL.match(l[0]))
        pos = j + 1
    out.extend(lines[pos:])
    return out


def _store_skips(blocks, loads):
    """Conditional branches that only skip stores: {block: lane-dependent}.

    The fall-through part of such a branch rejoins the branch target on
    every path and holds vector-memory stores but no untracked load.  A
    uniform branch of this kind is the inactive row (no prefetch in flight
    at its next wait); a branch on the execution mask is the wavefront none
    of whose lanes reaches the last chunk, which waits for one operation
    fewer."""
    out = {}
    for bi, (_, insts, succ) in enumerate(blocks):
        last = insts[-1][0] if insts else ""
        b = _BRANCH.match(last)
        if not (b and b.group(1).startswith("s_cbranch") and len(succ) == 2
                and succ[1] == bi + 1):
            continue
        target, seen, stack, closed = succ[0], set(), [bi + 1], True
        while stack and closed:
            x = stack.pop()
            if x == target or x in seen:
                continue
            if x == bi or not blocks[x][2]:
                closed = False
            seen.add(x)
            stack.extend(blocks[x][2])
        stores = any(_VMEM.match(t) and "store" in t for x in seen for t, _ in blocks[x][1])
        has_load = any((x, ii) in loads for x in seen for ii in range(len(blocks[x][1])))
        if closed and stores and not has_load:
            out[bi] = "exec" in b.group(1)
    return out


def _untracked_loads(blocks):
    loads = {}
    for bi, (_, insts, _) in enumerate(blocks):
        for ii, (text, in_asm) in enumerate(insts):
            m = _UNTRACKED.match(text) if in_asm else None
            if m:
                loads[(bi, ii)] = (set(range(int(m.group(1)), int(m.group(2)) + 1)), text.strip())
    return loads


def _flow(blocks, loads):
    """Violations found by following every path of the graph."""
    state_in = [frozenset() for _ in blocks]
    seen_in = [None] * len(blocks)
    violations, work = set(), [0]
    while work:
        bi = work.pop()
        if seen_in[bi] == state_in[bi]:
            continue
        seen_in[bi] = state_in[bi]
        state = set(state_in[bi])
        _, insts, succ = blocks[bi]
        for ii, (text, _) in enumerate(insts):
            key = (bi, ii)
            regs = _regs(text)
            if key in loads:
                regs = regs - loads[key][0]  # its own address, read at issue
            for lid, _n in state:
                if loads[lid][0] & regs:
                    violations.add((text.strip(), loads[lid][1]))
            if _VMEM.match(text):
                state = {(lid, min(n + 1, _CAP)) for lid, n in state}
            if key in loads:
                state.add((key, 0))
            w = _VMCNT.search(text) if text.strip().startswith("s_waitcnt") else None
            if w:
                state = {(lid, n) for lid, n in state if n < int(w.group(1))}
        out = frozenset(state)
        for s in succ:
            merged = state_in[s] | out
            if merged != state_in[s] or seen_in[s] is None:
                state_in[s] = merged
                work.append(s)
    return violations


def check_function(lines):
    """Violations (instruction text, load text) in one function, and the
    number of untracked loads it holds.

    Two executions are checked.  In the first every store runs and each
    wait region takes its weakest count; in the second each wavefront skips
    the stores of its last chunk (branches on the execution mask that only
    skip stores are taken) and each region takes its strongest count.  In
    both the row is active: uniform branches that only skip stores are not
    taken.  These are the two cases the kernels choose their counts for."""
    regions = _wait_regions(lines)
    violations, n_loads = set(), 0
    for pick, lane_skip in ((max, False), (min, True)):
        blocks = _blocks(_collapse(lines, regions, pick))
        loads = _untracked_loads(blocks)
        n_loads = len(loads)
        if not loads:
            return [], 0
        skips = _store_skips(blocks, loads)
        blocks = [(label, insts, ([succ[0]] if lane_skip and skips[bi] else [succ[1]])
                   if bi in skips else succ)
                  for bi, (label, insts, succ) in enumerate(blocks)]
        violations |= _flow(blocks, loads)
    return sorted(violations), n_loads


def explicit_waits(lines):
    """Indices of the wait instructions inside run-time wait regions."""
    return [q for i, j, _ in _wait_regions(lines) for q in range(i, j)
            if _VMCNT.search(lines[q][0]) and lines[q][0].strip().startswith("s_waitcnt")]


def check_listing(asm, name_filter=lambda name: True):
    """{function: (violations, untracked loads)} for the functions of a
    listing that hold untracked loads."""
    out = {}
    for name, lines in functions(asm).items():
        if not name_filter(name):
            continue
        violations, n = check_function(lines)
        if n:
            out[name] = (violations, n)
    return out
