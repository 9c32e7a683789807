"""Static check of the inline-assembly LDS reads in the deep-ring and four-wave GEMM kernels.

The kernels issue ds_read_b128 as inline assembly (so that the compiler does not drain the
global->LDS DMA ring before every LDS read) and wait for them themselves with
s_waitcnt lgkmcnt(0).  The compiler does not know that such a read writes its destination
registers later, so any instruction that reads or writes those registers before the wait would
see stale data or be overwritten.  This test walks the device assembly of the translation unit
(written by build() for every unit that has such reads) and checks, for every such read, that nothing but further inline LDS reads
touches its destination registers before an lgkmcnt(0) wait, and that no read is still pending
at a label or branch.  It needs no GPU."""
import os
import re

import pytest

BUILD = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                     "block_diffusion_drafter_draft_amd", "_build")
UNITS = ["k_gemm_deep.s"]

REG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")


def regs_of(text):
    out = set()
    for m in REG.finditer(text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _functions(lines):
    """Split device assembly into functions: name -> list of (line number, text, in_asm)."""
    fns, cur, in_asm = {}, None, False
    for no, raw in enumerate(lines, 1):
        t = raw.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        code = t.split(";")[0].strip()
        if not code:
            continue
        if code.endswith(":") and not code.startswith(".L") and not code.startswith("."):
            cur = code[:-1]
            fns[cur] = []
            continue
        if code.startswith(".Lfunc_end"):
            cur = None
            continue
        if cur is None or (code.startswith(".") and not code.endswith(":")):
            continue
        fns[cur].append((no, code, in_asm))
    return fns


def _blocks(body):
    """Basic blocks of one function: list of (label or None, instructions, successor labels,
    falls through)."""
    blocks, cur = [], [None, []]
    for no, code, in_asm in body:
        if code.endswith(":"):
            if cur[1] or cur[0] is not None:
                blocks.append(cur)
            cur = [code[:-1], []]
            continue
        cur[1].append((no, code, in_asm))
        op = code.split()[0]
        if op.startswith("s_cbranch") or op in ("s_branch", "s_endpgm", "s_setpc_b64"):
            blocks.append(cur)
            cur = [None, []]
    if cur[1] or cur[0] is not None:
        blocks.append(cur)
    out = []
    for lab, ins in blocks:
        succ, falls = [], True
        if ins:
            last = ins[-1][1].split()
            if last[0].startswith("s_cbranch"):
                succ.append(last[1])
            elif last[0] == "s_branch":
                succ.append(last[1])
                falls = False
            elif last[0] in ("s_endpgm", "s_setpc_b64"):
                falls = False
        out.append((lab, ins, succ, falls))
    return out


# The pending state is a map register -> age: the number of LDS operations issued after the
# read that writes it.  LDS operations complete in order, so s_waitcnt lgkmcnt(N) completes
# every read with N or more younger LDS operations.  Scalar memory operations also count on
# lgkmcnt but complete out of order: they never make a read older, so they are not counted.
MAX_AGE = 64


def _pending(state):
    return set(state)


def _age(state):
    return {r: min(a + 1, MAX_AGE) for r, a in state.items()}


def _step(state, no, code, in_asm, fn, bad):
    op = code.split()[0]
    if op == "s_waitcnt":
        m = re.search(r"lgkmcnt\((\d+)\)", code)
        if m:
            n = int(m.group(1))
            state = {r: a for r, a in state.items() if a < n}
        return state
    args = code.split(None, 1)[1] if " " in code else ""
    if in_asm and op == "ds_read_b128":
        dst, addr = args.split(",", 1)
        if regs_of(addr) & _pending(state):
            bad.add((fn, no, "address register of a pending read"))
        d = regs_of(dst)
        if d & _pending(state):
            bad.add((fn, no, "destination overlaps a pending read"))
        state = _age(state)
        for r in d:
            state[r] = 0
        return state
    if state and regs_of(args) & _pending(state):
        bad.add((fn, no, f"'{code[:60]}' touches a pending read's registers"))
    if op.startswith("ds_"):
        state = _age(state)          # any other LDS operation is younger than the reads
    return state


def _merge(into, new):
    """Join of two states: a register is pending if it is on either path, at the younger age."""
    changed = False
    for r, a in new.items():
        if r not in into or a < into[r]:
            into[r] = a
            changed = True
    return changed


def check(lines):
    """Dataflow over each function's control-flow graph: the registers of inline ds_read_b128
    not yet covered by an lgkmcnt wait, on any path, must not be read or written.  Returns a
    list of (function, line number, message)."""
    bad = set()
    for fn, body in _functions(lines).items():
        blocks = _blocks(body)
        index = {lab: k for k, (lab, _, _, _) in enumerate(blocks) if lab is not None}
        entry = [dict() for _ in blocks]
        work = list(range(len(blocks)))
        while work:
            k = work.pop(0)
            lab, ins, succ, falls = blocks[k]
            st = dict(entry[k])
            for no, code, in_asm in ins:
                st = _step(st, no, code, in_asm, fn, bad)
            nxt = [index[l] for l in succ if l in index]
            if falls and k + 1 < len(blocks):
                nxt.append(k + 1)
            for t in nxt:
                if _merge(entry[t], st) and t not in work:
                    work.append(t)
            if st and not nxt and ins and ins[-1][1].split()[0] == "s_endpgm":
                bad.add((fn, ins[-1][0], "program ends with pending reads"))
    return sorted(bad)


def test_checker_flags_a_planted_hazard():
    planted = ["kern:", ";;#ASMSTART", "ds_read_b128 v[4:7], v1", ";;#ASMEND",
               "v_add_u32_e32 v8, v5, v2", "s_waitcnt lgkmcnt(0)", "s_endpgm"]
    assert check(planted)
    # a hazard reached only through a branch
    branchy = ["kern:", ";;#ASMSTART", "ds_read_b128 v[4:7], v1", ";;#ASMEND",
               "s_cbranch_scc1 .LBB0_2", "s_waitcnt lgkmcnt(0)", "s_endpgm", ".LBB0_2:",
               "v_mov_b32_e32 v6, 0", "s_waitcnt lgkmcnt(0)", "s_endpgm"]
    assert check(branchy)
    # a partial wait covers the older read only
    partial = ["kern:", ";;#ASMSTART", "ds_read_b128 v[4:7], v1", ";;#ASMEND", ";;#ASMSTART",
               "ds_read_b128 v[8:11], v2", ";;#ASMEND", "s_waitcnt lgkmcnt(1)",
               "v_add_u32_e32 v20, v5, v2", "v_add_u32_e32 v21, v9, v2", "s_waitcnt lgkmcnt(0)",
               "s_endpgm"]
    bad = check(partial)
    assert len(bad) == 1 and bad[0][1] == 10
    clean = ["kern:", ";;#ASMSTART", "ds_read_b128 v[4:7], v1", ";;#ASMEND",
             "v_add_u32_e32 v8, v9, v2", "s_waitcnt lgkmcnt(0)", "v_add_u32_e32 v8, v5, v2",
             "s_endpgm"]
    assert not check(clean)


@pytest.mark.parametrize("unit", UNITS)
def test_inline_lds_reads_are_waited_for(unit):
    path = os.path.join(BUILD, unit)
    if not os.path.exists(path):
        pytest.skip("device assembly not built (run __graft_entry__.build())")
    lines = open(path).read().splitlines()
    n_reads = sum(1 for i, l in enumerate(lines) if "ds_read_b128" in l and i > 0
                  and lines[i - 1].strip().startswith(";;#ASMSTART"))
    assert n_reads > 0
    bad = check(lines)
    assert not bad, bad[:10]
