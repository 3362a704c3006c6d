"""Static check of gfx950 assembly for exponentials that sit in basic blocks
of their own.

A select such as `vis ? exp2(x) : 0` is not if-converted by the compiler
(the exponential counts as expensive): it becomes one exec-masked branch
per element, each guarding a block that holds little more than the
exponential.  This scanner splits every function at its block labels
(`.LBB...:` and the `; %bb.N:` markers of fall-through blocks) and reports
each block that contains a v_exp_f32 together with fewer than four other
vector instructions.  Test infrastructure only."""
from __future__ import annotations

import re

_FUNC = re.compile(r"^(_Z\w+):")
_BLOCK = re.compile(r"^(\.LBB\w+:|; %bb\.\d+:)")


def lone_exp_blocks(text: str) -> dict:
    """{function: [block label, ...]} for every block whose vector work is
    an exponential and at most three other vector instructions."""
    out: dict = {}
    func, label, n_exp, n_valu = None, None, 0, 0

    def close():
        if func is not None and n_exp and n_valu - n_exp < 4:
            out[func].append(label)

    for line in text.splitlines():
        m = _FUNC.match(line)
        if m:
            close()
            func, label, n_exp, n_valu = m.group(1), m.group(1), 0, 0
            out[func] = []
            continue
        if func is None:
            continue
        b = _BLOCK.match(line)
        if b:
            close()
            label, n_exp, n_valu = b.group(1), 0, 0
            continue
        tok = line.strip().split()
        if not tok:
            continue
        op = tok[0]
        if op == "s_endpgm":
            close()
            func = None
        elif op.startswith("v_"):
            n_valu += 1
            n_exp += op.startswith("v_exp_f32")
    close()
    return out
