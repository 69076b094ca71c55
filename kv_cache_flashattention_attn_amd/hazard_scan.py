"""Check the device assembly of libattn for MFMA results read too early across a branch.

An MFMA writes its result several cycles after it issues; a vector instruction that
reads the result must be at least that many wait states (instructions, or s_nop N
counting N + 1) behind it.  The compiler inserts the wait states reliably within a
basic block, but a read reached through a branch right after the MFMA has been seen
with too few: in one build of the decode kernel the row maximum read the last score
register one wait state after the MFMA that writes it, on the taken branch of the
length mask, while the same read within one block gets eight.  The result was a
stale maximum for one query head now and then (a non-repeatable output).

``scan(asm_text)`` follows every control-flow path from every MFMA to the first
vector instruction that reads one of its result registers and counts the wait
states.  For each MFMA opcode, the smallest count seen inside one basic block is
taken as the compiler's own requirement; a path that crosses a block boundary with
fewer is reported.  A path ends at an instruction that overwrites the result
registers first (a load, or another vector instruction writing them).  ``build.build()`` writes the assembly next to the library, and
tests/test_build_hazards.py runs this check on it.
"""
from __future__ import annotations

import re
import sys
from typing import Dict, List, Tuple

_ACCUMULATING = ("v_fmac", "v_dot2c", "v_mac", "v_fmamk", "v_fmaak")
# instructions whose first operand is a vector register they write (loads and
# vector ALU ops; comparisons and lane reads write scalar registers, which
# _regs ignores)
_WRITES_FIRST = ("v_", "global_load", "buffer_load", "flat_load", "scratch_load", "ds_read", "ds_bpermute",
                 "ds_swizzle")


def _regs(op: str) -> set:
    op = op.strip().rstrip(",").lstrip("-").strip("|")
    m = re.match(r"^v\[(\d+):(\d+)\]$", op)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"^v(\d+)$", op)
    return {int(m.group(1))} if m else set()


def _split(t: str) -> Tuple[str, List[str]]:
    parts = t.split(None, 1)
    args = [a.strip() for a in re.split(r",(?![^\[]*\])", parts[1])] if len(parts) > 1 else []
    return parts[0], args


def _kernels(text: str) -> Dict[str, List[str]]:
    out, cur = {}, None
    for ln in text.split("\n"):
        m = re.match(r"^(_Z\S+):", ln)
        if m:
            cur = m.group(1)
            out[cur] = []
            continue
        if cur is not None and re.match(r"^\.Lfunc_end", ln):
            cur = None
            continue
        if cur is not None:
            out[cur].append(ln)
    return out


def _blocks(body: List[str]):
    blocks, order, n = {"entry": []}, ["entry"], 0
    name = "entry"
    for ln in body:
        raw = ln.strip()
        mb = re.match(r"^; (%bb\.\d+):", raw)
        t = ln.split(";")[0].strip()
        ml = re.match(r"^(\.LBB\S+):", t)
        if mb or ml:
            name = ml.group(1) if ml else f"{mb.group(1)}#{n}"
            n += 1
            blocks[name] = []
            order.append(name)
            continue
        if not t or t.startswith("."):
            continue
        blocks[name].append(t)
        op = t.split()[0]
        if op.startswith("s_cbranch") or op == "s_branch":  # a branch ends the block
            name = f"#after{n}"
            n += 1
            blocks[name] = []
            order.append(name)
    succ = {}
    for i, b in enumerate(order):
        ins, s = blocks[b], []
        for t in ins:
            op = t.split()[0]
            if op.startswith("s_cbranch") or op == "s_branch":
                s.append(t.split()[1])
        last = ins[-1].split()[0] if ins else ""
        if last not in ("s_branch", "s_endpgm", "s_setpc_b64") and i + 1 < len(order):
            s.append(order[i + 1])
        succ[b] = [x for x in s if x in blocks]
    return blocks, order, succ


def _reads(body: List[str], limit: int = 40):
    """(mfma opcode, wait states, crossed a block boundary, kernel-local block, reader)."""
    blocks, order, succ = _blocks(body)
    found = []
    for b in order:
        for i, t in enumerate(blocks[b]):
            op, args = _split(t)
            if not op.startswith("v_mfma") or not args:
                continue
            dst = _regs(args[0])
            stack, seen = [(b, i + 1, 0, False, frozenset(dst))], set()
            while stack:
                state = stack.pop()
                if state in seen:
                    continue
                seen.add(state)
                bb, j, w, crossed, dst = state
                ins, done = blocks[bb], False
                live = set(dst)  # result registers not yet overwritten on this path
                while j < len(ins):
                    op2, a2 = _split(ins[j])
                    if op2.startswith("v_") and not op2.startswith("v_mfma"):
                        srcs = set().union(*[_regs(a) for a in a2[1:]]) if len(a2) > 1 else set()
                        if op2.startswith(_ACCUMULATING) and a2:
                            srcs |= _regs(a2[0])
                        if srcs & live:
                            found.append((op, w, crossed, bb, ins[j]))
                            done = True
                            break
                    if a2 and op2.startswith(_WRITES_FIRST):
                        live -= _regs(a2[0])  # a later write: the register no longer holds the result
                        if not live:
                            done = True
                            break
                    w += int(a2[0], 0) + 1 if op2 == "s_nop" else 1
                    if w > limit:
                        done = True
                        break
                    j += 1
                if not done:
                    for sb in succ[bb]:
                        stack.append((sb, 0, w, True, frozenset(live)))
    return found


def scan(text: str):
    """Returns (in-block minimum wait states per MFMA opcode, list of cross-block
    reads with fewer: (kernel, opcode, wait states, block, reader))."""
    per_kernel = {k: _reads(body) for k, body in _kernels(text).items()}
    need: Dict[str, int] = {}
    for found in per_kernel.values():
        for op, w, crossed, _, _ in found:
            if not crossed:
                need[op] = min(need.get(op, 1 << 30), w)
    bad = [(k, op, w, bb, t) for k, found in per_kernel.items() for op, w, crossed, bb, t in found
           if crossed and w < need.get(op, 0)]
    return need, bad


if __name__ == "__main__":
    need, bad = scan(open(sys.argv[1]).read())
    for op, w in sorted(need.items()):
        print(f"{op}: {w} wait states within a block")
    for k, op, w, bb, t in bad:
        print(f"EARLY READ {k[:80]}: {op} then {w} wait states to '{t}' ({bb})")
    print(f"{len(bad)} early cross-block reads")
    sys.exit(1 if bad else 0)
