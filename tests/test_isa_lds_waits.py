"""The device code that reads LDS through inline assembly never touches a
result before its lgkmcnt wait: compile each kernel source to gfx950
assembly with the library's own flags and scan it (no GPU needed).  The
scanner itself is pinned on hand-written listings with and without the
hazard."""
import os
import shutil
import subprocess

import pytest

from tests.isa_lds_check import check_asm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_sparse_msa_amd", "csrc")

GOOD = """_Zgood:
\tds_read_b64_tr_b16 v[4:5], v1 offset:0
\tds_read_b64_tr_b16 v[6:7], v1 offset:8
\ts_waitcnt lgkmcnt(1)
\tv_mov_b32 v8, v4
\ts_waitcnt lgkmcnt(0)
\tv_mov_b32 v9, v6
\ts_endpgm
"""
BAD = GOOD.replace("\ts_waitcnt lgkmcnt(1)\n\tv_mov_b32 v8, v4\n", "\ts_waitcnt lgkmcnt(1)\n\tv_mov_b32 v8, v6\n")


def test_scanner_accepts_ordered_waits():
    assert check_asm(GOOD) == {"_Zgood": []}


def test_scanner_flags_early_use():
    issues = check_asm(BAD)["_Zgood"]
    assert len(issues) == 1 and "pending [6]" in issues[0]


def _hipcc():
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.mark.parametrize("src", ["decode.hip", "attn_bf16.hip", "attn_bwd.hip", "attn_f32.hip", "pool.hip"])
def test_kernels_wait_before_use(src, tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    from long_context_sparse_msa_amd import build as b

    out = tmp_path / (src + ".s")
    cmd = [hipcc] + b.COMMON + b.EXTRA.get(src, []) + ["--cuda-device-only", "-S", os.path.join(CSRC, src),
                                                       "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    res = check_asm(out.read_text())
    assert res, "no functions found in the listing"
    bad = {f: i for f, i in res.items() if i}
    assert not bad, bad
