"""Check the compiled kernel for two hazards the hardware does not interlock.

The MFMAs of ``csrc/attn_fwd.hip`` are inline assembly, so the compiler does
not know they are MFMAs and pads them against neither rule of the MFMA
dependency table (CDNA3/CDNA4 ISA):
  * a VALU write of a VGPR or AGPR (``v_accvgpr_write``, ``v_mov``, any
    ``v_*`` result) needs at least two wait states before an MFMA reads that
    register as its A, B or C operand;
  * an MFMA result needs wait states before a VALU instruction reads it: 11
    or 12 for an 8-pass 32x32 MFMA, up to 20 for a 16-pass one; the check
    asks for 20.
The kernel is laid out so that neither happens; this module reads the
compiler's assembly and proves it, instruction by instruction, following
fall-through and every branch, backwards from each MFMA for the first rule and
forwards for the second. ``build.py`` runs it on every build and fails the
build on a violation.

(``v_readfirstlane``/``v_readlane`` are left out of the second rule: the
kernel never reads an MFMA result through them, and the compiler emits dead
ones that name an accumulator register as a placeholder source.)

Usage: ``python -m tiled_attention_16_amd.hazards kernel.s``
"""
from __future__ import annotations

import re
import sys
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Set, Tuple

WAIT_STATES = 2    # VALU write -> MFMA read of the same register
RESULT_WAIT = 20   # MFMA write -> VALU read of the same register

_REG = re.compile(r"^([va])(?:(\d+)|\[(\d+):(\d+)\])$")


def _regs(tok: str) -> Set[Tuple[str, int]]:
    m = _REG.match(tok.strip())
    if not m:
        return set()
    kind = m.group(1)
    if m.group(2) is not None:
        return {(kind, int(m.group(2)))}
    return {(kind, i) for i in range(int(m.group(3)), int(m.group(4)) + 1)}


@dataclass
class Ins:
    op: str
    args: List[str]
    line: int
    label: Optional[str] = None          # set on label pseudo-entries
    targets: List[str] = field(default_factory=list)


def _parse(text: str) -> List[List[Ins]]:
    """Split into functions; each a list of instructions and label entries."""
    funcs: List[List[Ins]] = []
    cur: Optional[List[Ins]] = None
    for n, raw in enumerate(text.split("\n"), 1):
        line = raw.split(";")[0].strip()
        if not line:
            continue
        if line.endswith(":") and not line.startswith("."):
            # a function symbol starts a new function body
            cur = []
            funcs.append(cur)
            continue
        if cur is None:
            continue
        if line.startswith(".LBB") and line.endswith(":"):
            cur.append(Ins("<label>", [], n, label=line[:-1]))
            continue
        if line.startswith("."):
            continue
        parts = line.split(None, 1)
        op = parts[0]
        args = [a.strip() for a in parts[1].split(",")] if len(parts) > 1 else []
        ins = Ins(op, args, n)
        if op.startswith("s_cbranch") or op == "s_branch":
            ins.targets = [a for a in args if a.startswith(".LBB")]
        cur.append(ins)
    return funcs


def _writes(ins: Ins) -> Set[Tuple[str, int]]:
    """Vector registers a VALU instruction writes (MFMAs excluded: the
    hardware orders MFMA -> MFMA accumulation itself)."""
    if not ins.op.startswith("v_") or ins.op.startswith("v_mfma") or ins.op.startswith("v_cmp"):
        return set()
    if not ins.args:
        return set()
    out = _regs(ins.args[0])
    if "permlane" in ins.op and "swap" in ins.op and len(ins.args) > 1:
        out |= _regs(ins.args[1])
    return out


def _wait_states(ins: Ins) -> int:
    if ins.op == "s_nop":
        return int(ins.args[0], 0) + 1 if ins.args else 1
    return 1


def _reads(ins: Ins) -> Set[Tuple[str, int]]:
    """Vector registers a VALU instruction reads (its source operands)."""
    if not ins.op.startswith("v_") or ins.op.startswith("v_mfma"):
        return set()
    if ins.op.startswith(("v_readfirstlane", "v_readlane")):
        return set()
    srcs = ins.args if ins.op.startswith("v_cmp") else ins.args[1:]
    out: Set[Tuple[str, int]] = set()
    for a in srcs:
        a = a.strip()
        if a.startswith("-"):
            a = a[1:]
        if a.startswith("|") and a.endswith("|"):
            a = a[1:-1]
        out |= _regs(a)
    if "permlane" in ins.op and "swap" in ins.op:
        out |= _regs(ins.args[0])
    return out


def check(text: str) -> List[str]:
    problems: List[str] = []
    for body in _parse(text):
        label_at: Dict[str, int] = {}
        branches_to: Dict[str, List[int]] = {}
        for i, ins in enumerate(body):
            if ins.label:
                label_at[ins.label] = i
            for t in ins.targets:
                branches_to.setdefault(t, []).append(i)

        def scan(i: int, need: int, reads: Set[Tuple[str, int]], seen: Set[Tuple[int, int]], where: int):
            # walk backwards from index i (exclusive) until `need` wait states are covered
            j = i - 1
            while need > 0:
                if j < 0:
                    return
                ins = body[j]
                if ins.label:
                    for b in branches_to.get(ins.label, []):
                        if (b, need) not in seen:
                            seen.add((b, need))
                            # the branch instruction itself is one wait state
                            scan(b, need - 1, reads, seen, where)
                    # fall-through predecessor: unless the previous instruction
                    # is an unconditional branch
                    if j > 0 and body[j - 1].op == "s_branch":
                        return
                    j -= 1
                    continue
                hit = _writes(ins) & reads
                if hit:
                    problems.append(f"line {where}: MFMA reads {sorted(hit)[0]} written by "
                                    f"'{ins.op} {', '.join(ins.args)}' (line {ins.line}) "
                                    f"with fewer than {WAIT_STATES} wait states between")
                    return
                need -= _wait_states(ins)
                j -= 1

        def scan_fwd(i: int, need: int, dst: Set[Tuple[str, int]], seen: Set[Tuple[int, int]], where: int):
            # walk forwards from index i (exclusive) until `need` wait states are covered
            j = i + 1
            while need > 0 and j < len(body):
                ins = body[j]
                if ins.label:
                    j += 1
                    continue
                if ins.op.startswith("v_mfma"):
                    if _regs(ins.args[0]) == dst:
                        return   # the accumulation chain continues; that MFMA is checked itself
                    need -= 1
                    j += 1
                    continue
                hit = _reads(ins) & dst
                if hit:
                    problems.append(f"line {ins.line}: '{ins.op} {', '.join(ins.args)}' reads {sorted(hit)[0]} "
                                    f"fewer than {RESULT_WAIT} wait states after the MFMA of line {where}")
                    return
                if ins.op == "s_endpgm":
                    return
                need -= _wait_states(ins)
                for t in ins.targets:
                    k = label_at.get(t)
                    if k is not None and (k, need) not in seen:
                        seen.add((k, need))
                        scan_fwd(k, need, dst, seen, where)
                if ins.op == "s_branch":
                    return
                j += 1

        for i, ins in enumerate(body):
            if not ins.op.startswith("v_mfma"):
                continue
            reads: Set[Tuple[str, int]] = set()
            for a in ins.args[1:4]:
                reads |= _regs(a)
            scan(i, WAIT_STATES, reads, set(), ins.line)
            scan_fwd(i, RESULT_WAIT, _regs(ins.args[0]), set(), ins.line)
    return problems


def main(argv: List[str]) -> int:
    text = open(argv[1]).read()
    probs = check(text)
    for p in probs:
        print(p)
    n = sum(1 for l in text.split("\n") if l.strip().startswith("v_mfma"))
    print(f"{n} MFMAs checked, {len(probs)} hazards")
    return 1 if probs else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
