"""Build libmsa.so (the C-ABI library with the gfx950 kernels) in-tree.

    python -m long_context_sparse_msa_amd.build

Every HIP source under csrc/ is compiled for gfx950 with hipcc and linked
into long_context_sparse_msa_amd/libmsa.so.  The measured references that
bench.py reports beside the kernels (ref/, not part of libmsa's interface)
go into libmsa_ref.so.  Packed-fp32 instruction selection is disabled for
all device code.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmsa.so")
REF_SRC = os.path.join(PKG, "ref", "mfma_ref.hip")
REF_LIB = os.path.join(PKG, "libmsa_ref.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (looked at $HIPCC, /opt/rocm/bin/hipcc, PATH)")


COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# Per-source extra flags.  The prefill kernel never relies on NaN semantics
# (NaN inputs give unspecified results), and without IEEE NaN handling the
# compiler drops the canonicalising max it otherwise puts in front of every
# max of an MFMA result.
EXTRA = {"attn_bf16.hip": ["-fno-honor-nans"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc()] + COMMON + EXTRA.get(os.path.basename(src), []) + ["-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines()
            if "packed-fp32-ops' is not a recognized feature" not in ln]
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build(verbose: bool = False) -> str:
    """Compile all sources and link libmsa.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    # A kernel whose host-side launch stub was not emitted leaves an
    # undefined stub symbol that only fails when the library is loaded with
    # eager binding; refuse such a link here.
    nm = shutil.which("nm") or "/usr/bin/nm"
    und = subprocess.run([nm, "-D", "--undefined-only", tmp], capture_output=True, text=True).stdout
    stubs = [ln.split()[-1] for ln in und.splitlines() if "__device_stub" in ln]
    if stubs:
        os.remove(tmp)
        raise RuntimeError("link left kernel launch stubs undefined: " + ", ".join(stubs))
    os.replace(tmp, LIB)
    build_ref()
    if verbose:
        print(f"built {LIB} and {REF_LIB}")
    return LIB


def build_ref() -> str:
    """Compile and link libmsa_ref.so (bench.py's measured references)."""
    tmp = REF_LIB + ".tmp"
    cmd = [hipcc()] + COMMON + ["-shared", REF_SRC, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {REF_SRC}:\n" + res.stdout + res.stderr)
    os.replace(tmp, REF_LIB)
    return REF_LIB


if __name__ == "__main__":
    build(verbose=True)
