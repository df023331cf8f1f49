"""Static check of the hazards that the forward kernels' inline assembly must avoid on gfx950.

The kernels issue their matrix-core products, and their transposed LDS reads, as inline assembly,
which the compiler's hazard recognizer and wait-count pass do not see into.  The rules they rely on,
checked here over the generated assembly of every kernel:

1. After a v_mfma writes its destination registers, no other instruction may read or write them for
   12 wait states (one per issued instruction, N+1 per s_nop N), 20 after the 16-pass fp8 product
   v_mfma_f32_32x32x64_f8f6f4 - except another v_mfma accumulating into exactly the same registers.
2. A VALU write of a register needs 2 wait states before a v_mfma reads it as an operand.
3. The destination of an LDS read (ds_read*, also when issued from inline assembly) is valid only
   after an s_waitcnt lgkmcnt(N) that covers it: LDS returns in order, so lgkmcnt(N) completes a
   read once N or more LDS instructions were issued after it.  Nothing may read or overwrite those
   registers before that.

The analysis is a forward data-flow pass over the instruction stream: the in-flight state is copied
at every branch, merged (union) at every label, and the pass runs twice so that states carried by
loop back edges reach the loop heads.

Usage: python check_mfma_hazards.py file.s [file.s ...]   (exit status 1 if a hazard is found)
"""
from __future__ import annotations

import re
import sys

MFMA_RESULT_WAIT = 12
MFMA_RESULT_WAIT_16PASS = 20  # 64-cycle products (the fp8 32x32x64 form)
VALU_TO_MFMA_WAIT = 2
REG = re.compile(r"\b([va])\[(\d+):(\d+)\]|\b([va])(\d+)\b")


def mfma_result_wait(op: str) -> int:
    return MFMA_RESULT_WAIT_16PASS if "32x32x64" in op or "16x16x128" in op else MFMA_RESULT_WAIT


def regs(text: str) -> frozenset:
    out = set()
    for m in REG.finditer(text):
        if m.group(1):
            for r in range(int(m.group(2)), int(m.group(3)) + 1):
                out.add((m.group(1), r))
        else:
            out.add((m.group(4), int(m.group(5))))
    return frozenset(out)


def split_operands(line: str):
    parts = line.split(None, 1)
    op = parts[0]
    ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
    return op, ops


def wait_states(op: str, ops) -> int:
    if op == "s_nop":
        try:
            return int(ops[0], 0) + 1
        except (ValueError, IndexError):
            return 1
    return 1


class State:
    """In-flight facts: MFMA results not yet safe, recent VALU writes, transposed reads not yet waited."""

    def __init__(self):
        self.mfma = {}  # (regs, dst operand, text) -> remaining wait states
        self.valu = {}  # (regs, text) -> remaining wait states
        self.tr = {}  # (regs, text) of LDS reads -> LDS instructions issued after it (minimum over paths)

    def copy(self):
        s = State()
        s.mfma, s.valu, s.tr = dict(self.mfma), dict(self.valu), dict(self.tr)
        return s

    def merge(self, other: "State"):
        for k, v in other.mfma.items():
            self.mfma[k] = max(v, self.mfma.get(k, 0))
        for k, v in other.valu.items():
            self.valu[k] = max(v, self.valu.get(k, 0))
        for k, v in other.tr.items():
            self.tr[k] = min(v, self.tr.get(k, v))


def functions(path: str):
    """(name, [(lineno, instruction or label)]) for every function in the file."""
    name, body = None, []
    for lineno, raw in enumerate(open(path), 1):
        line = raw.split(";")[0].strip()
        if not line:
            continue
        if line.endswith(":") and not line.startswith("."):
            if name is not None:
                yield name, body
            name, body = line[:-1], []
            continue
        if line.startswith(".") and not line.endswith(":"):
            continue  # directive
        if name is not None:
            body.append((lineno, line))
    if name is not None:
        yield name, body


def check_function(path: str, name: str, body) -> list:
    problems = set()
    label_pos = {line[:-1]: i for i, (_, line) in enumerate(body) if line.endswith(":")}
    incoming = {}  # label -> merged state of the branches to it
    for _ in range(2):
        state = State()
        for lineno, line in body:
            if line.endswith(":"):
                lab = line[:-1]
                if lab in incoming:
                    if state is None:
                        state = incoming[lab].copy()
                    else:
                        state.merge(incoming[lab])
                if state is None:
                    state = State()
                continue
            if state is None:
                continue  # unreachable
            op, ops = split_operands(line)
            if op.startswith("s_cbranch") or op == "s_branch":
                tgt = ops[0] if ops else None
                if tgt in label_pos:
                    if tgt in incoming:
                        incoming[tgt].merge(state)
                    else:
                        incoming[tgt] = state.copy()
                if op == "s_branch":
                    state = None
                continue
            if op == "s_endpgm":
                state = None
                continue
            if op == "s_waitcnt":
                m = re.search(r"lgkmcnt\((\d+)\)", line)
                if m:
                    n = int(m.group(1))
                    state.tr = {k: v for k, v in state.tr.items() if v < n}
                continue
            touched = regs(line)
            is_mfma = op.startswith("v_mfma")
            # rule 1
            for (wr, dst, text), rem in state.mfma.items():
                hit = wr & touched
                if hit and not (is_mfma and ops and ops[0] == dst and len(ops) > 3 and ops[3] == dst):
                    problems.add(f"{path}:{lineno}: {name}: '{line}' touches {sorted(hit)[:2]} written by "
                                 f"'{text}' {mfma_result_wait(text.split()[0]) - rem} wait states earlier")
            # rule 2
            if is_mfma and len(ops) > 1:
                srcs = frozenset().union(*[regs(o) for o in ops[1:]])
                for (wr, text), rem in state.valu.items():
                    hit = wr & srcs
                    if hit:
                        problems.add(f"{path}:{lineno}: {name}: '{line}' reads {sorted(hit)[:2]} written by "
                                     f"VALU '{text}' {VALU_TO_MFMA_WAIT - rem} wait states earlier")
            # rule 3
            for (wr, text), _n in state.tr.items():
                hit = wr & touched
                if hit:
                    problems.add(f"{path}:{lineno}: {name}: '{line}' touches {sorted(hit)[:2]} before the "
                                 f"transposed read '{text}' is known complete")
            ws = wait_states(op, ops)
            state.mfma = {k: r - ws for k, r in state.mfma.items() if r - ws > 0}
            state.valu = {k: r - ws for k, r in state.valu.items() if r - ws > 0}
            if op.startswith("ds_"):
                state.tr = {k: v + 1 for k, v in state.tr.items()}
            if is_mfma and ops:
                state.mfma[(regs(ops[0]), ops[0], line)] = mfma_result_wait(op)
            elif op.startswith("v_") and ops:
                state.valu[(regs(ops[0]), line)] = VALU_TO_MFMA_WAIT
            if op.startswith("ds_read") and ops:
                state.tr[(regs(ops[0]), line)] = 0
    return sorted(problems)


def check(path: str) -> list:
    out = []
    for name, body in functions(path):
        out += check_function(path, name, body)
    return out


def main(argv) -> int:
    bad = []
    for path in argv:
        bad += check(path)
    for p in bad[:40]:
        print(p)
    print(f"{len(bad)} hazards in {len(argv)} file(s)")
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
