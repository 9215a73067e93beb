"""Checks on the gfx950 assembly of the decode kernels, run by the build.

The decode kernels with three or four waves accumulate O block 15 with an inline-asm
VGPR-form `v_mfma_f32_32x32x16_bf16` whose latency the compiler cannot see: until the
drain (three `s_nop 7`) after the tile loop, the MFMA may still be writing its registers.
The code is only correct if no other instruction touches those registers in that window
(a register copy, a spill or a read by the compiler would see a partly written block).
`vgpr_mfma_violations` checks that on the compiler's output:

1. in a kernel, every VGPR-form MFMA accumulates in place into one 16-register range R;
2. on every control-flow path, between such an MFMA and the next drain, no instruction
   other than those MFMAs names a register of R.

Rule 2 is a forward dataflow over the kernel's basic blocks (split at labels and after
branches): the state "an MFMA may be in flight" is set by the MFMA, cleared by the drain
and joined over predecessors until it no longer changes, so loop back edges and blocks
laid out out of order are covered.
"""

from __future__ import annotations

import re

_FUNC = re.compile(r"^(_Z\S+):")
_LABEL = re.compile(r"^(\.LBB\d+_\d+):")
_BRANCH = re.compile(r"^\s*s_(?:c?branch)\S*\s+(\.LBB\d+_\d+)")
_VMFMA = re.compile(r"^\s*v_mfma_f32_32x32x16_bf16\s+v\[(\d+):(\d+)\],\s*v\[\d+:\d+\],\s*v\[\d+:\d+\],\s*v\[(\d+):(\d+)\]")
_VREG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")


def _instructions(lines):
    """(kind, text) items of one function: kind is 'label' or 'insn'; comments dropped."""
    out = []
    for raw in lines:
        m = _LABEL.match(raw)
        if m:
            out.append(("label", m.group(1)))
            continue
        text = raw.split(";", 1)[0].rstrip()
        if not text.strip() or text.lstrip().startswith("."):
            continue
        if raw[:1] in (" ", "\t"):
            out.append(("insn", text.strip()))
    return out


def _functions(asm: str):
    funcs, name, body = {}, None, []
    for line in asm.splitlines():
        m = _FUNC.match(line)
        if m:
            name, body = m.group(1), []
            funcs[name] = body
            continue
        if name is not None:
            if line.startswith(".Lfunc_end"):
                name = None
                continue
            body.append(line)
    return funcs


def _touches(insn: str, lo: int, hi: int) -> bool:
    parts = insn.split(None, 1)
    if len(parts) < 2:
        return False
    for m in _VREG.finditer(parts[1]):
        a, b = (int(m.group(1)), int(m.group(2))) if m.group(1) else (int(m.group(3)), int(m.group(3)))
        if a <= hi and b >= lo:
            return True
    return False


def _blocks(items):
    """Basic blocks: (labels, instructions, successor block indices)."""
    blocks, cur_labels, cur = [], [], []

    def close():
        nonlocal cur_labels, cur
        if cur_labels or cur:
            blocks.append([cur_labels, cur])
        cur_labels, cur = [], []

    for kind, t in items:
        if kind == "label":
            if cur:
                close()
            cur_labels.append(t)
            continue
        cur.append(t)
        if t.startswith("s_branch") or t.startswith("s_cbranch") or t.startswith("s_endpgm") \
                or t.startswith("s_setpc") or t.startswith("s_trap"):
            close()
    close()
    where = {lab: i for i, (labs, _) in enumerate(blocks) for lab in labs}
    out = []
    for i, (labs, body) in enumerate(blocks):
        last = body[-1] if body else ""
        succ = []
        m = _BRANCH.match(last)
        if last.startswith("s_branch") and m:
            succ = [where[m.group(1)]] if m.group(1) in where else []
        elif last.startswith("s_cbranch") and m:
            succ = ([where[m.group(1)]] if m.group(1) in where else []) + ([i + 1] if i + 1 < len(blocks) else [])
        elif last.startswith("s_endpgm") or last.startswith("s_setpc") or last.startswith("s_trap"):
            succ = []
        elif i + 1 < len(blocks):
            succ = [i + 1]
        out.append((labs, body, succ))
    return out


def _is_drain(body, k):
    return k >= 2 and all(body[k - j] == "s_nop 7" for j in range(3))


def vgpr_mfma_violations(asm: str) -> list:
    """Messages naming each breach of the rules above; empty when the code is safe."""
    problems = []
    for fname, lines in _functions(asm).items():
        items = _instructions(lines)
        ranges = set()
        for kind, t in items:
            m = _VMFMA.match(t) if kind == "insn" else None
            if m:
                d0, d1, c0, c1 = map(int, m.groups())
                ranges.add((d0, d1))
                if (d0, d1) != (c0, c1) or d1 - d0 != 15:
                    problems.append(f"{fname}: VGPR-form MFMA not accumulating in place over 16 registers: {t}")
        if not ranges:
            continue
        if len(ranges) != 1:
            problems.append(f"{fname}: VGPR-form MFMAs use {len(ranges)} accumulator ranges {sorted(ranges)}")
            continue
        lo, hi = next(iter(ranges))
        blocks = _blocks(items)

        def transfer(body, state, report=None):
            for k, t in enumerate(body):
                if _VMFMA.match(t):
                    state = True
                elif _is_drain(body, k):
                    state = False
                elif state and report is not None and _touches(t, lo, hi):
                    report.append(f"{fname}: v[{lo}:{hi}] named while the MFMA may be in flight: {t}")
            return state

        n = len(blocks)
        in_state, out_state = [False] * n, [False] * n
        preds = [[] for _ in range(n)]
        for i, (_, _, succ) in enumerate(blocks):
            for j in succ:
                preds[j].append(i)
        changed = True
        while changed:
            changed = False
            for i, (_, body, _) in enumerate(blocks):
                st = any(out_state[p] for p in preds[i])
                o = transfer(body, st)
                if st != in_state[i] or o != out_state[i]:
                    in_state[i], out_state[i], changed = st, o, True
        for i, (_, body, _) in enumerate(blocks):
            transfer(body, in_state[i], problems)
    return problems


def count_vgpr_mfma_kernels(asm: str) -> int:
    """Functions holding at least one VGPR-form MFMA (to see that the check had work)."""
    return sum(1 for lines in _functions(asm).values()
               if any(_VMFMA.match(t) for k, t in _instructions(lines) if k == "insn"))
