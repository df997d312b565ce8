"""Checks on compiled AMDGPU assembly for the MFMAs written as inline
assembly (the tied-accumulator 16x16x32 form).  The compiler's hazard
recognizer does not see those as MFMAs, so the kernel source promises:

  1. after such an MFMA, no other instruction reads or writes an AGPR until a
     drain (four `s_nop 7`) has executed, on every control-flow path;
  2. after a non-MFMA write of an AGPR, no such MFMA until a drain;
  3. no VALU instruction writes a VGPR that such an MFMA reads as its A or B
     operand within 4 wait states before it (also across block boundaries).

`check_function` verifies all three on the text `clang -S` emits, where each
inline-assembly statement sits between `;;#ASMSTART` and `;;#ASMEND`.

The buffer-descriptor loads into LDS share one M0 write among the loads of
a 4 KiB LDS group: a load that does not write M0 itself relies on the group's
first load having done so, with nothing writing M0 in between.
`check_m0` verifies that M0 is written only by inline assembly and that on
every path to such a load the last M0 write came from inline assembly.
Test infrastructure only; nothing here is part of the product path."""
import re

_AGPR = re.compile(r"\ba(?:\d+|\[\d+:\d+\])")
_BRANCH = re.compile(r"s_(?:cbranch_\w+|branch)\s+(\.LBB\S+)")


def functions(asm_text: str):
    """Yield (symbol, lines) for every function in an assembly listing."""
    lines = asm_text.split("\n")
    i = 0
    while i < len(lines):
        m = re.match(r"^(_Z\S+):", lines[i])
        if not m:
            i += 1
            continue
        j = i
        while j < len(lines) and not lines[j].startswith(".Lfunc_end"):
            j += 1
        yield m.group(1), lines[i:j]
        i = j


def _blocks(lines, tag_asm=False):
    blocks, cur, in_asm = [], [None, []], False
    for line in lines:
        m = re.match(r"^(\.LBB\S+):", line)
        if m:
            if cur[0] is not None or cur[1]:
                blocks.append(cur)
            cur = [m.group(1), []]
            continue
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not line.startswith("\t") or not t or t.startswith(";") or t.startswith("."):
            continue
        t = t.split(";")[0].strip()
        if in_asm and t.startswith("v_mfma"):
            t = "ASM " + t
        elif in_asm and tag_asm:
            t = "INL " + t
        cur[1].append(t)
        if t.startswith(("s_branch", "s_cbranch", "s_endpgm", "s_setpc")):
            blocks.append(cur)
            cur = [None, []]
    if cur[0] is not None or cur[1]:
        blocks.append(cur)
    index = {b[0]: k for k, b in enumerate(blocks) if b[0]}
    succ, pred = [[] for _ in blocks], [[] for _ in blocks]
    for k, (_, ins) in enumerate(blocks):
        last = ins[-1] if ins else ""
        m = _BRANCH.match(last)
        if m:
            succ[k].append(index[m.group(1)])
        if not last.startswith(("s_branch", "s_endpgm", "s_setpc")) and k + 1 < len(blocks):
            succ[k].append(k + 1)
    for k, ss in enumerate(succ):
        for s in ss:
            pred[s].append(k)
    return blocks, succ, pred


def _operands(t):
    parts = t.split(None, 1)
    return [x.strip() for x in parts[1].split(",")] if len(parts) > 1 else []


def _vgprs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _wait_states(t):
    m = re.match(r"s_nop\s+(\d+)$", t)
    return int(m.group(1)) + 1 if m else 1


def check_function(lines):
    """Return (number of inline-asm MFMAs, list of rule violations)."""
    blocks, succ, pred = _blocks(lines)
    n_asm = sum(1 for _, ins in blocks for t in ins if t.startswith("ASM "))
    violations = []

    # rules 1 and 2: forward dataflow of (MFMA pending, AGPR write pending)
    def step(k, state, record):
        mfma, write = state
        nops = 0
        for t in blocks[k][1]:
            if t == "s_nop 7":
                nops += 1
                if nops >= 4:
                    mfma = write = False
                continue
            nops = 0
            if t.startswith("ASM "):
                if write and record:
                    violations.append(("AGPR write, then MFMA without a drain", t))
                mfma = True
                continue
            if t.startswith("v_mfma"):
                continue
            ops = _operands(t)
            if any(_AGPR.search(o) for o in ops):
                if mfma and record:
                    violations.append(("AGPR access after an MFMA without a drain", t))
                if ops and _AGPR.match(ops[0]) and not t.startswith(("scratch_store", "buffer_store", "global_store", "ds_write")):
                    write = True
        return mfma, write

    state_in = [(False, False)] * len(blocks)
    changed = True
    while changed:
        changed = False
        for k in range(len(blocks)):
            out = step(k, state_in[k], False)
            for s in succ[k]:
                new = (state_in[s][0] or out[0], state_in[s][1] or out[1])
                if new != state_in[s]:
                    state_in[s] = new
                    changed = True
    for k in range(len(blocks)):
        step(k, state_in[k], True)

    # rule 3: backward search from each inline-asm MFMA over 4 wait states
    def writes_vgpr(t, regs):
        if not t.startswith("v_") or t.startswith(("v_mfma", "v_cmp", "v_readfirstlane", "v_readlane")):
            return False
        ops = _operands(t)
        return bool(ops) and bool(_vgprs(ops[0]) & regs)

    def search(k, pos, regs, budget, seen):
        ins = blocks[k][1]
        for q in range(pos - 1, -1, -1):
            if writes_vgpr(ins[q], regs):
                return ins[q]
            budget -= _wait_states(ins[q])
            if budget <= 0:
                return None
        for p in pred[k]:
            if (p, budget) in seen:
                continue
            seen.add((p, budget))
            hit = search(p, len(blocks[p][1]), regs, budget, seen)
            if hit:
                return hit
        return None

    for k, (_, ins) in enumerate(blocks):
        for q, t in enumerate(ins):
            if not t.startswith("ASM "):
                continue
            ops = _operands(t[4:])
            regs = set().union(*(_vgprs(o) for o in ops[1:3]))
            hit = search(k, q, regs, 4, set())
            if hit:
                violations.append(("VALU write of an MFMA source within 4 wait states", hit + " -> " + t))
    return n_asm, violations


def _writes_m0(t):
    ops = _operands(t)
    return bool(ops) and ops[0] == "m0"


def check_m0(lines):
    """Return (number of inline-assembly LDS-DMA loads checked, list of
    violations): M0 written outside inline assembly, or a load reached on
    some path with no inline-assembly M0 write as the last write of M0."""
    blocks, succ, pred = _blocks(lines, tag_asm=True)
    violations, relying = [], 0

    def step(k, ours, record):
        nonlocal relying
        for t in blocks[k][1]:
            inl = t.startswith("INL ")
            body = t[4:] if inl else t
            if _writes_m0(body):
                if not inl and record:
                    violations.append(("M0 written outside inline assembly", body))
                ours = inl
                continue
            if inl and re.match(r"(?:global_load_lds_\w+\s|buffer_load_\w+ .*\blds$)", body):
                if record:
                    relying += 1
                    if not ours:
                        violations.append(("LDS-DMA load without an inline-assembly M0 write before it", body))
        return ours

    # forward dataflow: "the last M0 write on every path came from inline
    # assembly"; false at the entry (M0 is undefined there)
    state_in = [True] * len(blocks)
    if blocks:
        state_in[0] = False
    changed = True
    while changed:
        changed = False
        for k in range(len(blocks)):
            inc = state_in[k] if k == 0 else all(step(p, state_in[p], False) for p in pred[k]) if pred[k] else state_in[k]
            if k == 0:
                inc = False
            if inc != state_in[k]:
                state_in[k] = inc
                changed = True
    for k in range(len(blocks)):
        step(k, state_in[k], True)
    return relying, violations
