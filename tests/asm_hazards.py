"""Wait-state checks on gfx950 assembly of kernels that issue matrix-core
operations from inline asm (which the compiler's hazard recognizer cannot see
into).

Two rules, each checked over every control-flow path into the consumer:
  - a VALU instruction that writes a VGPR or AccVGPR read by a v_mfma (its A,
    B or C operand) must be followed by at least 2 wait states before it;
  - a v_mfma result must not be read or overwritten by any other instruction
    (an AccVGPR read or move, for instance) within RESULT_WAIT wait states.
    The compiler pads 8 after a 16x16x64 INT8 operation (four passes) before
    a VALU read; RESULT_WAIT keeps a margin of 2 over that.
A wait state is one issued instruction; s_nop N counts N + 1. Branch
instructions count 0 (conservative).
"""
import re

RESULT_WAIT = 10

_REG = re.compile(r"\b([va])(\d+)\b|\b([va])\[(\d+):(\d+)\]")


def _regs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(1):
            out.add((m.group(1), int(m.group(2))))
        else:
            for r in range(int(m.group(4)), int(m.group(5)) + 1):
                out.add((m.group(3), r))
    return out


def _split_ops(rest):
    ops, depth, cur = [], 0, ""
    for ch in rest:
        if ch == "[":
            depth += 1
        elif ch == "]":
            depth -= 1
        if ch == "," and depth == 0:
            ops.append(cur.strip())
            cur = ""
        else:
            cur += ch
    if cur.strip():
        ops.append(cur.strip())
    return ops


class _Insn:
    __slots__ = ("line", "mn", "ops", "text", "label", "cost", "writes", "reads")

    def __init__(self, line, text, label=None):
        self.line, self.text, self.label = line, text, label
        self.mn, self.ops, self.cost = "", [], 0
        self.writes, self.reads = set(), set()
        if label is not None:
            return
        parts = text.split(None, 1)
        self.mn = parts[0]
        self.ops = _split_ops(parts[1]) if len(parts) > 1 else []
        if self.mn == "s_nop":
            self.cost = int(self.ops[0], 0) + 1
        elif self.mn.startswith(("s_branch", "s_cbranch")):
            self.cost = 0
        else:
            self.cost = 1
        vector = self.mn.startswith("v_")
        if vector and self.ops and not self.mn.startswith(("v_cmp", "v_readlane", "v_readfirstlane")):
            self.writes = _regs(self.ops[0])
            self.reads = set().union(*(_regs(o) for o in self.ops[1:])) if len(self.ops) > 1 else set()
        else:
            # memory and scalar instructions: every vector register named is read
            # (loads write their first operand, which no rule here consumes)
            self.reads = set().union(*(_regs(o) for o in self.ops)) if self.ops else set()

    @property
    def is_valu(self):
        return self.mn.startswith("v_") and not self.mn.startswith("v_mfma")

    @property
    def is_mfma(self):
        return self.mn.startswith("v_mfma")


def _functions(asm_text):
    """{function name: [_Insn]} for the functions defined in asm_text."""
    funcs, cur, name = {}, None, None
    for ln, raw in enumerate(asm_text.splitlines(), 1):
        line = raw.split(";")[0].strip()
        if not line or line.startswith((".", "//")) and not re.match(r"^\.L\w+:", line):
            continue
        m = re.match(r"^([.\w$]+):$", line)
        if m:
            lab = m.group(1)
            if lab.startswith(".Lfunc_end"):
                cur = None  # the function's code ends here (it may hold several s_endpgm)
                continue
            if not lab.startswith("."):
                name = lab
                cur = funcs.setdefault(name, [])
            if cur is not None:
                cur.append(_Insn(ln, line, label=lab))
            continue
        if cur is not None:
            cur.append(_Insn(ln, line))
    return funcs


def _walk_back(insns, idx, branches_to, need, hit, ws=0, seen=None):
    """Visit the instructions before insns[idx] on every path, while fewer than
    `need` wait states separate them from it; hit(insn, ws) returns True to
    stop that path."""
    if seen is None:
        seen = set()
    i = idx - 1
    while i >= 0 and ws < need:
        ins = insns[i]
        if ins.label is not None:
            for b in branches_to.get(ins.label, ()):
                if (b, ws) not in seen:
                    seen.add((b, ws))
                    _walk_back(insns, b + 1, branches_to, need, hit, ws, seen)
            prev = insns[i - 1] if i > 0 else None
            if prev is not None and prev.label is None and prev.mn in ("s_branch", "s_endpgm", "s_setpc_b64"):
                return
            i -= 1
            continue
        if hit(ins, ws):
            return
        ws += ins.cost
        i -= 1


def check(asm_text, name_filter):
    """Returns (number of v_mfma checked, [problem strings]) over the functions
    whose name contains name_filter."""
    problems, n_mfma = [], 0
    for fname, insns in _functions(asm_text).items():
        if name_filter not in fname:
            continue
        branches_to = {}
        for i, ins in enumerate(insns):
            if ins.mn.startswith(("s_branch", "s_cbranch")) and ins.ops:
                branches_to.setdefault(ins.ops[-1], []).append(i)
        for i, ins in enumerate(insns):
            if ins.label is not None:
                continue
            if ins.is_mfma:
                n_mfma += 1
                srcs = set().union(*(_regs(o) for o in ins.ops[1:4]))

                def hit(p, ws, srcs=srcs, ins=ins):
                    if p.is_valu and p.writes & srcs and ws < 2:
                        problems.append(f"{fname}:{ins.line}: {p.mn} (line {p.line}) writes an operand of "
                                        f"'{ins.text}' {ws} wait states before it")
                    return False

                _walk_back(insns, i, branches_to, 2, hit)
            touched = (ins.reads | ins.writes) if not ins.is_mfma else set()
            aregs = {r for r in touched if r[0] == "a"}
            if aregs:
                def hit2(p, ws, aregs=aregs, ins=ins):
                    if p.is_mfma and _regs(p.ops[0]) & aregs:
                        problems.append(f"{fname}:{ins.line}: '{ins.text}' touches the result of "
                                        f"'{p.text}' (line {p.line}) {ws} wait states after it")
                        return True
                    return False

                _walk_back(insns, i, branches_to, RESULT_WAIT, hit2)
    return n_mfma, problems
