"""MI355X-native causal sliding-window + mean-pooled-landmark sparse attention.

The compute lives in libmsa.so (C ABI in include/msa.h, gfx950 HIP kernels
under csrc/); this package is its thin Python binding.
"""
from .binding import (  # noqa: F401
    EXPORTS,
    MSA_DECODE_AUTO,
    MSA_DECODE_FUSED,
    MSA_DECODE_SPLIT,
    MSA_DTYPE_BF16,
    MSA_DTYPE_F32,
    AttnDesc,
    DecodeDesc,
    MsaError,
    abi_version,
    attn_desc,
    decode_desc,
    decode_partials,
    lib,
    msa_append_kv,
    msa_attn_bwd,
    msa_attn_bwd_workspace_size,
    msa_attn_fwd,
    msa_attn_fwd_blocksparse,
    msa_append_kv_paged,
    msa_decode_fwd,
    msa_decode_fwd_noalloc,
    msa_decode_fwd_paged,
    msa_decode_fwd_varlen,
    msa_decode_workspace_size,
    msa_plan_decode,
    msa_plan_decode_varlen,
    msa_plan_rows,
    msa_plan_tiles,
    msa_pool_landmarks,
)

pool_landmarks = msa_pool_landmarks
attn_fwd = msa_attn_fwd
attn_bwd = msa_attn_bwd
attn_fwd_blocksparse = msa_attn_fwd_blocksparse
decode_fwd = msa_decode_fwd
decode_fwd_varlen = msa_decode_fwd_varlen
append_kv = msa_append_kv
