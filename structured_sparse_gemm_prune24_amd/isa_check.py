"""Build-time check of the GEMM kernels' final gfx950 assembly.

The kernels issue their LDS fragment reads as inline assembly so that the
compiler does not insert its own conservative waits; a read's destination
registers then only hold the data after the `s_waitcnt lgkmcnt` that covers it,
while the compiler treats them as written at issue.  Any instruction that reads
(or overwrites) such a register before that wait -- typically a register copy
the compiler adds -- works on stale data, and the result depends on timing.

`pending_lds_uses(asm)` follows the control flow of every kernel of a device
assembly file and reports those instructions.  LDS operations complete in issue
order, so `s_waitcnt lgkmcnt(N)` leaves only the newest N LDS / scalar-memory
operations in flight; the analysis keeps that queue per instruction, merging the
queues of all paths that reach it (a loop's back edge included) until nothing
changes.  The merge takes, position by position from the newest end, the union
of the pending registers, so it over-reports rather than misses.
"""
from __future__ import annotations

import re
from typing import Dict, List, Tuple

_KERNEL = re.compile(r"\n(_ZN3p246k_gemm\S+):[^\n]*\n(.*?)\.Lfunc_end", re.S)
_STORES = ("ds_write", "global_store", "buffer_store", "flat_store", "scratch_store")


def _vregs(tok: str) -> set:
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _operands(line: str) -> Tuple[str, List[str]]:
    op = line.split()[0]
    rest = line[len(op):]
    return op, [o.strip().split()[0] for o in rest.split(",") if o.strip()]


_MAX_QUEUE = 256     # a longer queue (no wait at all in a loop) collapses into one pending set


def _merge(a: List[set], b: List[set]) -> List[set]:
    """Queues aligned at their newest end, unioned position by position."""
    if len(a) < len(b):
        a, b = b, a
    out = list(a)
    off = len(a) - len(b)
    for k, regs in enumerate(b):
        out[off + k] = out[off + k] | regs
    return out


def _step(line: str, queue: List[set]) -> Tuple[List[set], bool]:
    """Effect of one instruction on the in-flight queue; True if it touches a pending register."""
    op, ops = _operands(line)
    pending = set().union(*queue) if queue else set()
    if op == "s_waitcnt":
        m = re.search(r"lgkmcnt\((\d+)\)", line)
        if m:
            queue = queue[max(0, len(queue) - int(m.group(1))):]
        return queue, False
    if op.startswith("ds_"):
        is_read = op.startswith("ds_read") or op.startswith("ds_bpermute") or op.startswith("ds_permute")
        dst = _vregs(ops[0]) if (ops and is_read) else set()
        srcs = set().union(*(_vregs(o) for o in (ops[1:] if is_read else ops))) if ops else set()
        queue = queue + [dst]
        if len(queue) > _MAX_QUEUE:
            queue = [set().union(*queue)]
        return queue, bool(srcs & pending)
    if op.startswith(("s_load", "s_buffer_load", "s_memtime", "s_memrealtime")):
        return queue + [set()], False
    if op.startswith("s_"):
        return queue, False
    is_store = op.startswith(_STORES)
    srcs = set().union(*(_vregs(o) for o in (ops if is_store else ops[1:]))) if ops else set()
    dst = set() if is_store or not ops else _vregs(ops[0])
    return queue, bool((srcs | dst) & pending)


def _flow(body: str) -> Tuple[List[str], List[List[int]]]:
    """Instructions of a kernel body and the successors of each (branch targets, fall-through)."""
    instrs: List[str] = []
    labels: Dict[str, int] = {}
    for raw in body.split("\n"):
        line = raw.split(";")[0].strip()
        if not line or line.startswith("."):
            if line.endswith(":"):
                labels[line[:-1]] = len(instrs)
            continue
        if line.endswith(":"):
            labels[line[:-1]] = len(instrs)
            continue
        instrs.append(line)
    succ: List[List[int]] = []
    for i, line in enumerate(instrs):
        op = line.split()[0]
        nxt = [i + 1] if i + 1 < len(instrs) else []
        if op == "s_branch":
            succ.append([labels[line.split()[1]]])
        elif op.startswith("s_cbranch"):
            succ.append(nxt + [labels[line.split()[1]]])
        elif op in ("s_endpgm", "s_setpc_b64"):
            succ.append([])
        else:
            succ.append(nxt)
    return instrs, succ


def pending_lds_uses(asm: str) -> Dict[str, List[str]]:
    """Kernel name -> instructions that touch a VGPR with an LDS read still in flight."""
    out: Dict[str, List[str]] = {}
    for name, body in _KERNEL.findall(asm):
        instrs, succ = _flow(body)
        if not instrs:
            continue
        state: Dict[int, List[set]] = {0: []}
        work = [0]
        while work:
            i = work.pop()
            q, _ = _step(instrs[i], state[i])
            for j in succ[i]:
                old = state.get(j)
                new = q if old is None else _merge(old, q)
                if old is None or new != old:
                    state[j] = new
                    work.append(j)
        bad = [instrs[i] for i in sorted(state) if _step(instrs[i], state[i])[1]]
        if bad:
            out[name] = bad
    return out


def spilling_kernels(asm: str) -> List[str]:
    """Kernels that touch scratch memory (register spills).  The loop's hand-counted
    vmcnt waits stay correct with extra memory operations in flight (they only get
    stricter), but a spill inside the loop costs a memory round trip per step."""
    return [name for name, body in _KERNEL.findall(asm) if re.search(r"^\s*scratch_", body, re.M)]


def check_file(path: str) -> None:
    with open(path) as f:
        asm = f.read()
    found = pending_lds_uses(asm)
    if found:
        lines = [f"{k}: {len(v)} (first: {v[0]})" for k, v in found.items()]
        raise RuntimeError(f"{path}: instructions use LDS read results before their wait:\n" + "\n".join(lines))
    spills = spilling_kernels(asm)
    if spills:
        raise RuntimeError(f"{path}: GEMM kernels spill registers to scratch:\n" + "\n".join(spills))
