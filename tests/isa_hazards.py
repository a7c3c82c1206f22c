"""Static check of our own gfx950 assembly: every path from an MFMA to the first
VALU / memory instruction that reads its destination must carry at least
`min_gap` wait states (one per instruction, N+1 per `s_nop N`), following both
fall-through and taken branches.  The compiler pads straight-line code with at
least 10 wait states after a 16x16x4 f32 MFMA; a path with fewer (for example a
taken branch straight into the read) returns a stale accumulator.
"""
import re


def _regs(tok):
    m = re.fullmatch(r'([av])(\d+)', tok)
    if m:
        return {tok}
    m = re.fullmatch(r'([av])\[(\d+):(\d+)\]', tok)
    if m:
        return {f"{m.group(1)}{r}" for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    return set()


def _parse(line):
    line = line.split(';')[0].strip()
    if not line:
        return None
    parts = line.split(None, 1)
    ops = [o.strip() for o in parts[1].split(',')] if len(parts) > 1 else []
    return parts[0], ops


def functions(asm_text):
    return re.findall(r'^(_Z\w+):[^\n]*\n(.*?)\.Lfunc_end', asm_text, flags=re.S | re.M)


def short_paths(asm_text, min_gap=10):
    """List (function, mfma index, reading instruction, wait states) for every violation."""
    found = []
    for name, body in functions(asm_text):
        instr, lab = [], {}
        for raw in body.splitlines():
            t = raw.strip()
            if t.startswith('.LBB'):
                lab[t.split(':')[0]] = len(instr)
                continue
            if not t or t.startswith(('.', ';')):
                continue
            p = _parse(t)
            if p:
                instr.append(p)
        for i, (op, ops) in enumerate(instr):
            if not op.startswith('v_mfma') or not ops:
                continue
            dst = _regs(ops[0])
            stack, seen = [(i + 1, 0)], set()
            while stack:
                j, gap = stack.pop()
                while j < len(instr) and gap < min_gap:
                    if (j, gap) in seen:
                        break
                    seen.add((j, gap))
                    o, a = instr[j]
                    if o == 's_nop':
                        gap += int(a[0]) + 1
                        j += 1
                        continue
                    if o.startswith('v_mfma'):  # chained MFMAs forward their accumulator
                        gap += 1
                        j += 1
                        continue
                    store = o.startswith(('global_store', 'buffer_store', 'ds_write', 'flat_store'))
                    srcs = set()
                    for x in (a if store else a[1:]):
                        if x:
                            srcs |= _regs(x.split()[0])
                    if o.startswith(('v_', 'global_', 'ds_', 'buffer_', 'flat_')) and srcs & dst:
                        found.append((name, i, o, gap))
                        break
                    if o.startswith('s_cbranch') or o == 's_branch':
                        if a and a[0] in lab:
                            stack.append((lab[a[0]], gap + 1))
                        if o == 's_branch':
                            break
                    if o == 's_endpgm':
                        break
                    gap += 1
                    j += 1
    return found
