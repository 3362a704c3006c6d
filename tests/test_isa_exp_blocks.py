"""No kernel forms its exponentials one divergent branch per element:
compile each kernel source to gfx950 assembly with the library's own
flags and look for blocks that hold an exponential and little else (no GPU
needed).  The scanner is pinned on hand-written listings first."""
import os
import shutil
import subprocess

import pytest

from tests.isa_exp_check import lone_exp_blocks

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_sparse_msa_amd", "csrc")

# the softmax of a tile in one block: exponentials among the other vector work
GOOD = """_Zgood:
\tv_fma_f32 v1, v2, s4, v3
\tv_fma_f32 v5, v6, s4, v3
\tv_exp_f32_e32 v1, v1
\tv_exp_f32_e32 v5, v5
\tv_add_f32_e32 v7, v1, v5
\tv_cvt_pk_bf16_f32 v8, v1, v5
\tv_sub_f32_e32 v9, v10, v11
\ts_endpgm
"""
# the same element by element behind exec-masked branches
BAD = """_Zbad:
\ts_and_saveexec_b64 s[0:1], vcc
\ts_cbranch_execz .LBB0_2
; %bb.1:
\tv_fma_f32 v1, v2, s4, v3
\tv_exp_f32_e32 v1, v1
.LBB0_2:
\ts_or_b64 exec, exec, s[0:1]
\ts_and_saveexec_b64 s[0:1], vcc
\ts_cbranch_execz .LBB0_4
; %bb.3:
\tv_fma_f32 v5, v6, s4, v3
\tv_exp_f32_e32 v5, v5
.LBB0_4:
\ts_or_b64 exec, exec, s[0:1]
\tv_add_f32_e32 v7, v1, v5
\ts_endpgm
"""


def test_scanner_accepts_softmax_block():
    assert lone_exp_blocks(GOOD) == {"_Zgood": []}


def test_scanner_flags_branch_per_element():
    assert lone_exp_blocks(BAD) == {"_Zbad": ["; %bb.1:", "; %bb.3:"]}


def _hipcc():
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.mark.parametrize("src", ["decode.hip", "attn_bf16.hip", "attn_bwd.hip", "attn_f32.hip"])
def test_no_exponential_per_branch(src, tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    from long_context_sparse_msa_amd import build as b

    out = tmp_path / (src + ".s")
    cmd = [hipcc] + b.COMMON + b.EXTRA.get(src, []) + ["--cuda-device-only", "-S", os.path.join(CSRC, src),
                                                       "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    res = lone_exp_blocks(out.read_text())
    assert res, "no functions found in the listing"
    bad = {f: blocks for f, blocks in res.items() if blocks}
    assert not bad, bad
