"""Use-before-wait check of LDS reads in generated gfx950 assembly.

The kernels issue their MFMA operand reads from LDS as inline assembly and wait for
them with explicit s_waitcnt lgkmcnt(n). The compiler sees such a read's result as
ready at once, so nothing but the scheduling fences keeps it from placing a consumer
(an MFMA, a copy) above the wait. This scan tracks, in program order, the LDS
operations outstanding per lgkmcnt and reports any instruction that touches a
register whose LDS read has not been waited for. Straight-line tracking: across a
label the outstanding list is carried over, which only errs on the strict side for
code whose reads and waits sit in one block.
"""
from __future__ import annotations

import re

_RANGE = re.compile(r"v\[(\d+):(\d+)\]")
_SINGLE = re.compile(r"v(\d+)$")


def _regs(tok: str) -> set[int]:
    m = _RANGE.match(tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = _SINGLE.match(tok)
    return {int(m.group(1))} if m else set()


def violations(asm_text: str) -> list[str]:
    found = []
    kernel = "?"
    pending: list[set[int]] = []  # outstanding LDS operations, oldest first (destination registers)
    for ln, line in enumerate(asm_text.splitlines(), 1):
        s = line.split(";")[0].strip()
        if re.match(r"^_Z\w+:", s):
            kernel, pending = s[:-1], []
            continue
        if not s or s.startswith(".") or s.endswith(":"):
            continue
        parts = s.replace(",", " ").split()
        op = parts[0]
        if op == "s_waitcnt":
            m = re.search(r"lgkmcnt\((\d+)\)", s)
            if m:
                n = int(m.group(1))
                pending = pending[len(pending) - n:] if n < len(pending) else pending
            continue
        live = set().union(*pending) if pending else set()
        if op.startswith("ds_"):
            srcs = set().union(*[_regs(t) for t in parts[2:]]) if op.startswith(("ds_read", "ds_load")) else \
                set().union(*[_regs(t) for t in parts[1:]])
            if srcs & live:
                found.append(f"line {ln} in {kernel}: {s}")
            pending.append(_regs(parts[1]) if op.startswith(("ds_read", "ds_load")) else set())
            continue
        if op.startswith("s_") or op.startswith("global_load_lds"):
            continue
        used = set().union(*[_regs(t) for t in parts[1:]])
        if used & live:
            found.append(f"line {ln} in {kernel}: {s}")
    return found
