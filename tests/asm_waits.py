"""Dataflow check of hand-issued loads in gfx950 device assembly.

The weight-streaming GEMM issues some global and LDS loads itself (inline asm) and waits
for them with s_waitcnt statements whose comment names the registers they cover ("waits
for v[4:7]").  The compiler sees such a load's destination as written when the statement
ends, so the code is only sound if, along every path of the control-flow graph, no
instruction reads a register whose hand-issued load may still be in flight (other than the
naming wait), and none writes one (the load could land after it).  A full vmcnt(0) /
lgkmcnt(0) without a name retires everything.
"""
from __future__ import annotations

import re

_REG = re.compile(r'([va])\[(\d+):(\d+)\]|([va])(\d+)$')


def _regs(tok: str) -> set[str]:
    tok = tok.strip().split()[0] if tok.strip() else ''
    m = re.match(r'([va])\[(\d+):(\d+)\]', tok)
    if m:
        return {f'{m.group(1)}{i}' for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r'([va])(\d+)$', tok)
    return {tok} if m else set()


def _blocks(lines: list[str]):
    blocks, cur, in_asm = [], {'label': 'entry', 'ins': []}, False
    for raw in lines:
        st = raw.strip()
        if st.startswith(';;#ASMSTART'):
            in_asm = True
            continue
        if st.startswith(';;#ASMEND'):
            in_asm = False
            continue
        m = re.match(r'^(\.LBB\w+):', st)
        if m or st.startswith('; %bb.'):
            blocks.append(cur)
            cur = {'label': m.group(1) if m else st, 'ins': []}
            continue
        if not st or st.startswith((';', '.')):
            continue
        cur['ins'].append((st, in_asm))
    blocks.append(cur)
    return blocks


def check_function(lines: list[str]) -> list[str]:
    """Violations in one function's assembly lines."""
    blocks = _blocks(lines)
    index = {b['label']: i for i, b in enumerate(blocks)}
    succ = []
    for i, b in enumerate(blocks):
        s = [index[m.group(1)] for ins, _ in b['ins'] for m in [re.match(r's_c?branch\w*\s+(\.LBB\w+)', ins)] if m]
        last = b['ins'][-1][0] if b['ins'] else ''
        if not last.startswith(('s_branch', 's_endpgm')) and i + 1 < len(blocks):
            s.append(i + 1)
        succ.append(s)
    state = [None] * len(blocks)
    state[0] = (frozenset(), frozenset())
    work, viol = [0], set()
    while work:
        i = work.pop()
        vm, lg = set(state[i][0]), set(state[i][1])
        for ins, hand in blocks[i]['ins']:
            op = ins.split()[0]
            text, _, comment = ins.partition(';')
            args = text[len(op):].split(',')
            if op == 's_waitcnt':
                m = re.search(r'waits for (\S+)', comment)
                named = _regs(m.group(1)) if m else set()
                if 'vmcnt(0)' in ins and not named:
                    vm = set()
                if 'lgkmcnt(0)' in ins and not named:
                    lg = set()
                if 'vmcnt' in ins:
                    vm -= named
                if 'lgkmcnt' in ins:
                    lg -= named
                continue
            used = set()
            for a in args:
                used |= _regs(a)
            dst = _regs(args[0]) if args and args[0].strip() else set()
            live = vm | lg
            where = f"{blocks[i]['label']}: {ins[:90]}"
            if hand and op.startswith('global_load') and not op.startswith('global_load_lds'):
                if (used - dst) & live or dst & live:
                    viol.add('load over an in-flight register: ' + where)
                vm |= dst
                continue
            if hand and op.startswith('ds_read'):
                if used & live:
                    viol.add('LDS read over an in-flight register: ' + where)
                lg |= dst
                continue
            if used & live:
                viol.add('reads or writes an in-flight register: ' + where)
        out = (frozenset(vm), frozenset(lg))
        for j in succ[i]:
            new = out if state[j] is None else (state[j][0] | out[0], state[j][1] | out[1])
            if new != state[j]:
                state[j] = new
                work.append(j)
    return sorted(viol)


def check_assembly(text: str, name_pattern: str) -> dict[str, list[str]]:
    """Violations per function whose symbol matches name_pattern."""
    out = {}
    for name in re.findall(rf'^({name_pattern}\w*):', text, re.M):
        start = text.index(name + ':')
        end = text.index('.Lfunc_end', start)
        out[name] = check_function(text[start:end].split('\n')[1:])
    return out
