"""The hot kernels keep their working set in registers: compile each kernel
source to gfx950 assembly with the library's own flags and read the code
object metadata (no GPU needed).  A spill puts scratch loads and stores in
the tile loop, and every scratch load's wait also waits for the tiles that
are still streaming into LDS, so the prefetch stops hiding anything."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_sparse_msa_amd", "csrc")

# kernels that must not spill at all
NO_SPILL = ("attn_fwd_bf16_kernel", "attn_fwd_list_kernel", "bwd_dq_kernel", "bwd_dkdv_kernel",
            "decode_fused_kernel", "decode_split_kernel", "decode_merge_kernel", "pool_kernel", "append_kernel")


def kernel_registers(text: str) -> dict:
    """{kernel name: (vgpr_count, vgpr_spill_count)} from the AMDGPU
    metadata block of an assembly listing."""
    out = {}
    for entry in re.split(r"\n\s*- \.agpr_count:", text)[1:]:
        name = re.search(r"\.name:\s+(\S+)", entry)
        vg = re.search(r"\.vgpr_count:\s+(\d+)", entry)
        sp = re.search(r"\.vgpr_spill_count:\s+(\d+)", entry)
        if name and vg and sp:
            out[name.group(1)] = (int(vg.group(1)), int(sp.group(1)))
    return out


LISTING = """
amdhsa.kernels:
  - .agpr_count:     0
    .name:           _ZN3msa12_GLOBAL__N_120attn_fwd_bf16_kernelILi128ELb1EEEvv
    .vgpr_count:     198
    .vgpr_spill_count: 0
  - .agpr_count:     0
    .name:           _ZN3msa12_GLOBAL__N_115bwd_dkdv_kernelILi128ELb0ELb1EEEvv
    .vgpr_count:     256
    .vgpr_spill_count: 3
"""


def test_parser_reads_metadata():
    regs = kernel_registers(LISTING)
    assert regs == {"_ZN3msa12_GLOBAL__N_120attn_fwd_bf16_kernelILi128ELb1EEEvv": (198, 0),
                    "_ZN3msa12_GLOBAL__N_115bwd_dkdv_kernelILi128ELb0ELb1EEEvv": (256, 3)}


def _hipcc():
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.mark.parametrize("src", ["attn_bf16.hip", "attn_bwd.hip", "decode.hip", "pool.hip"])
def test_hot_kernels_do_not_spill(src, tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    from long_context_sparse_msa_amd import build as b

    out = tmp_path / (src + ".s")
    cmd = [hipcc] + b.COMMON + b.EXTRA.get(src, []) + ["--cuda-device-only", "-S", os.path.join(CSRC, src),
                                                       "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    regs = kernel_registers(out.read_text())
    assert regs, "no kernel metadata found in the listing"
    for name, (vgprs, spills) in regs.items():
        assert vgprs <= 256, (name, vgprs)
        if any(k in name for k in NO_SPILL):
            assert spills == 0, (name, spills)
