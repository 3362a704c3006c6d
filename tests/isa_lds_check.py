"""Static check of gfx950 assembly for LDS-read results used before an
lgkmcnt wait covers them.

Kernels that issue ds_read_b64_tr_b16 as inline assembly wait for the
results with explicit `s_waitcnt lgkmcnt(n)`; the compiler does not know
those reads are asynchronous, so a copy or use it schedules between a read
and its wait would see stale registers.  This scanner walks each function
linearly, keeps the destination registers of outstanding LDS reads in
issue order (LDS operations complete in order), retires them at every
lgkmcnt wait, and reports any instruction that reads or overwrites a
register still pending.  It is deliberately conservative (straight-line,
loop back-edges ignored, SMEM ignored) and is test infrastructure only."""
from __future__ import annotations

import re

_REG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")
_FUNC = re.compile(r"^(_Z\w+):")
_WAIT = re.compile(r"s_waitcnt\b.*lgkmcnt\((\d+)\)")


def _regs(text: str) -> set:
    out = set()
    for m in _REG.finditer(text):
        if m.group(3):
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def check_function(lines):
    """lines: [(line_no, text)] of one function.  Returns a list of issues."""
    pending = []  # destination register sets of outstanding LDS operations, oldest first
    issues = []
    for ln, raw in lines:
        t = raw.split(";")[0].strip()
        if not t or t.endswith(":") or t.startswith("."):
            continue
        op = t.split()[0]
        parts = [a.strip() for a in t[len(op):].split(",") if a.strip()]
        m = _WAIT.match(t)
        if m:
            n = int(m.group(1))
            while len(pending) > n:
                pending.pop(0)
            continue
        live = set().union(*pending) if pending else set()
        if op.startswith("ds_"):
            is_read = op.startswith("ds_read")
            srcs = set().union(*[_regs(a) for a in (parts[1:] if is_read else parts)]) if parts else set()
            if srcs & live:
                issues.append(f"{ln}: {t}  reads pending {sorted(srcs & live)}")
            pending.append(_regs(parts[0]) if is_read and parts else set())
            continue
        if op == "s_endpgm":
            pending = []
            continue
        if not parts:
            continue
        if op.startswith(("buffer_store", "global_store", "global_load_lds", "buffer_load")):
            srcs = set().union(*[_regs(a) for a in parts])
            dst = set()
        else:
            srcs = set().union(*[_regs(a) for a in parts[1:]]) if len(parts) > 1 else set()
            dst = _regs(parts[0]) if not op.startswith("s_") else set()
        if srcs & live:
            issues.append(f"{ln}: {t}  reads pending {sorted(srcs & live)}")
        if dst & live:
            issues.append(f"{ln}: {t}  overwrites pending {sorted(dst & live)}")
    return issues


def check_asm(text: str) -> dict:
    """{function name: [issues]} for every function in an assembly listing."""
    funcs, cur = {}, None
    for i, line in enumerate(text.splitlines(), 1):
        m = _FUNC.match(line)
        if m:
            cur = m.group(1)
            funcs[cur] = []
        elif cur is not None:
            funcs[cur].append((i, line))
    return {f: check_function(ls) for f, ls in funcs.items()}
