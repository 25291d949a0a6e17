"""Build-time check of the GEMM kernels' final gfx950 assembly.

The kernels issue their LDS fragment reads as inline assembly so that the
compiler does not insert its own conservative waits; a read's destination
registers then only hold the data after the `s_waitcnt lgkmcnt` that covers it,
while the compiler treats them as written at issue.  Any instruction that reads
(or overwrites) such a register before that wait -- typically a register copy
the compiler adds -- works on stale data, and the result depends on timing.

`pending_lds_uses(asm)` scans every kernel of a device assembly file in program
order and reports those instructions.  LDS operations complete in issue order,
so `s_waitcnt lgkmcnt(N)` leaves only the newest N LDS / scalar-memory
operations in flight; the scan keeps that queue.  It is linear: a branch does
not reset what is pending, so it over-reports rather than misses.
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


def pending_lds_uses(asm: str) -> Dict[str, List[str]]:
    """Kernel name -> instructions that touch a VGPR with an LDS read still in flight."""
    out: Dict[str, List[str]] = {}
    for name, body in _KERNEL.findall(asm):
        queue: List[set] = []        # in-flight LDS / scalar-memory operations, oldest first (read destinations)
        bad: List[str] = []
        for raw in body.split("\n"):
            line = raw.split(";")[0].strip()
            if not line or line.endswith(":") or line.startswith("."):
                continue
            op, ops = _operands(line)
            pending = set().union(*queue) if queue else set()
            if op == "s_waitcnt":
                m = re.search(r"lgkmcnt\((\d+)\)", line)
                if m:
                    n = int(m.group(1))
                    del queue[:max(0, len(queue) - n)]
                continue
            if op.startswith("ds_"):
                is_read = op.startswith("ds_read") or op.startswith("ds_bpermute") or op.startswith("ds_permute")
                dst = _vregs(ops[0]) if (ops and is_read) else set()
                srcs = set().union(*(_vregs(o) for o in (ops[1:] if is_read else ops))) if ops else set()
                if srcs & pending:
                    bad.append(line)
                queue.append(dst)
                continue
            if op.startswith(("s_load", "s_buffer_load", "s_memtime", "s_memrealtime")):
                queue.append(set())
                continue
            if op.startswith("s_"):
                continue
            is_store = op.startswith(_STORES)
            srcs = set().union(*(_vregs(o) for o in (ops if is_store else ops[1:]))) if ops else set()
            dst = set() if is_store or not ops else _vregs(ops[0])
            if (srcs | dst) & pending:
                bad.append(line)
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
