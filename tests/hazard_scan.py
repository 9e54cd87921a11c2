"""Control-flow-aware check of matrix-core result hazards in gfx950 device assembly.

An MFMA writes its destination registers a fixed number of wait states after it issues, and
the hardware does not hold back a later instruction that reads them sooner: the compiler
must put enough independent instructions or s_nop between the two.  It does so along code
as laid out, but a branch that skips a region (s_cbranch_execz over a masked block) can
reach the first reader along a shorter path.  For every MFMA this module walks every path
forward through the kernel's branches and records the fewest wait states (one per
instruction, N + 1 per s_nop N) before an instruction that reads one of its result
registers that no other instruction has overwritten since.  Reads that follow the layout
give the wait the compiler enforces; paths through a taken branch must not be shorter.
"""
from __future__ import annotations

import heapq
import re
from collections import defaultdict

_REG = re.compile(r"([va])\[(\d+):(\d+)\]|([va])(\d+)")
_LOADS = ("ds_read", "ds_bpermute", "global_load", "buffer_load", "flat_load", "scratch_load")
_MEM = ("ds_", "global_", "buffer_", "flat_", "scratch_")


def _regs(op: str) -> frozenset:
    m = _REG.fullmatch(op)
    if not m:
        return frozenset()
    if m.group(1):
        return frozenset((m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1))
    return frozenset({(m.group(4), int(m.group(5)))})


def _parse(line: str):
    parts = line.split(None, 1)
    ops = [o.strip().split()[0] for o in parts[1].split(",") if o.strip()] if len(parts) > 1 else []
    return parts[0], ops


def kernels(asm_text: str) -> dict:
    """Function name -> list of ('label', name) / ('ins', text), in layout order."""
    out, cur = {}, None
    for raw in asm_text.splitlines():
        m = re.match(r"^([A-Za-z_][\w.$]*):", raw)
        if m and not raw.startswith(".L"):
            cur = m.group(1)
            out[cur] = []
            continue
        if cur is None:
            continue
        t = raw.strip()
        if t.startswith(".Lfunc_end"):
            cur = None
        elif re.match(r"^\.LBB\w*:", t):
            out[cur].append(("label", t.split(":")[0]))
        elif t and not t.startswith((".", ";")):
            out[cur].append(("ins", t.split(";")[0].strip()))
    return out


def _reads_writes(opc: str, ops: list):
    """Registers an instruction reads and writes (vector and accumulator registers)."""
    reads, writes = set(), set()
    for k, op in enumerate(ops):
        r = _regs(op)
        if k == 0 and (opc.startswith(_LOADS) or (opc.startswith("v_") and not opc.startswith(
                ("v_cmp", "v_readlane", "v_readfirstlane")))):
            writes |= r
        else:
            reads |= r
    return reads, writes


def scan(body: list, limit: int = 40):
    """(mfma opcode, reader kind, wait states, via a taken branch) for every MFMA result
    read within `limit` wait states of the MFMA, over all paths."""
    ins, labels = [], {}
    for kind, text in body:
        if kind == "label":
            labels[text] = len(ins)
        else:
            ins.append(_parse(text))

    def succ(i):
        opc, ops = ins[i]
        if opc in ("s_endpgm", "s_setpc_b64"):
            return []
        if opc == "s_branch":
            return [labels[ops[0]]] if ops and ops[0] in labels else []
        nxt = [i + 1] if i + 1 < len(ins) else []
        if opc.startswith("s_cbranch") and ops and ops[0] in labels:
            nxt.append(labels[ops[0]])
        return nxt

    def wait_states(i):
        opc, ops = ins[i]
        return int(ops[0], 0) + 1 if opc == "s_nop" and ops else 1

    found = []
    for i, (opc, ops) in enumerate(ins):
        if not opc.startswith("v_mfma") or not ops:
            continue
        dst = _regs(ops[0])
        heap = [(0, j, j != i + 1, dst) for j in succ(i)]
        seen = {}
        steps = 0
        while heap and steps < 50000:
            d, j, branched, live = heapq.heappop(heap)
            steps += 1
            if d >= limit or not live:
                continue
            if seen.get((j, branched, live), limit + 1) <= d:
                continue
            seen[(j, branched, live)] = d
            o2, ops2 = ins[j]
            if o2.startswith("v_mfma"):
                if len(ops2) > 3 and _regs(ops2[0]) == live and _regs(ops2[3]) == live:
                    continue  # the accumulation chain goes on: its last product is checked
                if any(_regs(x) & live for x in ops2[1:3]):
                    found.append((opc, "mfma operand", d, branched))
                writes = _regs(ops2[0])
            elif o2.startswith(("v_",) + _MEM):
                reads, writes = _reads_writes(o2, ops2)
                if reads & live:
                    found.append((opc, "vector or memory", d, branched))
                    continue
            else:
                writes = set()
            rest = frozenset(live - writes)
            for s in succ(j):
                heapq.heappush(heap, (d + wait_states(j), s, branched or s != j + 1, rest))
    return found


def summarise(asm_texts) -> dict:
    """(mfma opcode, reader kind) -> [fewest wait states along the layout, through a branch]."""
    out = defaultdict(lambda: [None, None])
    for text in asm_texts:
        for body in kernels(text).values():
            for opc, kind, d, branched in scan(body):
                slot = out[(opc, kind)]
                k = 1 if branched else 0
                slot[k] = d if slot[k] is None else min(slot[k], d)
    return dict(out)
