"""Thin Python binding of libmsa's C ABI (include/msa.h).

Argument marshalling only: shapes and dtypes are read off torch tensors,
outputs are allocated with torch when not given, and the call is forwarded
to the library on the tensors' current HIP stream.  Every step of the
computation runs in libmsa's kernels; there is no fallback path, and
loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmsa.so")

MSA_OK = 0
MSA_ERR_INVALID_ARG = 1
MSA_ERR_UNSUPPORTED = 2
MSA_ERR_WORKSPACE = 3
MSA_ERR_HIP = 4
MSA_ERR_CAPACITY = 5

MSA_DTYPE_F32 = 0
MSA_DTYPE_BF16 = 1

EXPORTS = (
    "msa_pool_landmarks", "msa_attn_fwd", "msa_decode_workspace_size", "msa_decode_fwd",
    "msa_plan_rows", "msa_plan_tiles", "msa_plan_decode", "msa_status_string",
    "msa_last_error", "msa_abi_version", "msa_decode_fwd_varlen", "msa_append_kv",
    "msa_plan_decode_varlen", "msa_attn_bwd_workspace_size", "msa_attn_bwd", "msa_attn_fwd_blocksparse",
    "msa_decode_fwd_paged", "msa_append_kv_paged", "msa_decode_fwd_noalloc",
)

LIST_QUERY_BLOCK = 128
LIST_KEY_BLOCK = 64


class MsaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libmsa status {status}: {msg}")
        self.status = status


class AttnDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
                ("seq_len", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("window", ctypes.c_int32),
                ("num_landmarks", ctypes.c_int32), ("scale", ctypes.c_float),
                ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32)]


class DecodeDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
                ("ctx_len", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("window", ctypes.c_int32),
                ("num_landmarks", ctypes.c_int32), ("num_splits", ctypes.c_int32),
                ("scale", ctypes.c_float), ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("schedule", ctypes.c_int32)]


MSA_DECODE_AUTO = 0
MSA_DECODE_SPLIT = 1
MSA_DECODE_FUSED = 2
_SCHEDULES = {None: MSA_DECODE_AUTO, "auto": MSA_DECODE_AUTO, "split": MSA_DECODE_SPLIT, "fused": MSA_DECODE_FUSED}


def _schedule_code(schedule) -> int:
    if isinstance(schedule, int):
        return schedule
    if schedule not in _SCHEDULES:
        raise ValueError(f"schedule must be one of {sorted(k for k in _SCHEDULES if k)} (got {schedule!r})")
    return _SCHEDULES[schedule]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libmsa (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: build it with "
                              "`python -m long_context_sparse_msa_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        P = ctypes.POINTER
        L.msa_pool_landmarks.argtypes = [P(AttnDesc), vp, vp, vp, vp, vp]
        L.msa_attn_fwd.argtypes = [P(AttnDesc), vp, vp, vp, vp, vp, vp, vp, vp]
        L.msa_decode_workspace_size.argtypes = [P(DecodeDesc), P(sz)]
        L.msa_decode_fwd.argtypes = [P(DecodeDesc), vp, vp, vp, vp, vp, vp, sz, vp, vp, vp]
        L.msa_plan_rows.argtypes = [P(AttnDesc), vp, vp]
        L.msa_plan_tiles.argtypes = [P(AttnDesc), vp, i64, P(i64), P(i32), P(i32)]
        L.msa_plan_decode.argtypes = [P(DecodeDesc), vp, P(i32), P(i32)]
        L.msa_decode_fwd_varlen.argtypes = [P(DecodeDesc), vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp]
        L.msa_append_kv.argtypes = [P(DecodeDesc), vp, vp, vp, vp, vp, vp, vp, vp]
        L.msa_plan_decode_varlen.argtypes = [P(DecodeDesc), i32, vp, P(i32), P(i32)]
        L.msa_attn_bwd_workspace_size.argtypes = [P(AttnDesc), P(sz)]
        L.msa_attn_fwd_blocksparse.argtypes = [P(AttnDesc), vp, vp, i32, i32, vp, vp, vp, vp, vp, vp]
        L.msa_decode_fwd_paged.argtypes = [P(DecodeDesc), i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp]
        L.msa_append_kv_paged.argtypes = [P(DecodeDesc), i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.msa_attn_bwd.argtypes = [P(AttnDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp, vp]
        L.msa_decode_fwd_noalloc.argtypes = [P(DecodeDesc), vp, vp, vp, vp, vp, vp, vp, vp]
        for f in ("msa_pool_landmarks", "msa_attn_fwd", "msa_decode_workspace_size", "msa_decode_fwd",
                  "msa_plan_rows", "msa_plan_tiles", "msa_plan_decode", "msa_decode_fwd_varlen",
                  "msa_append_kv", "msa_plan_decode_varlen", "msa_attn_bwd_workspace_size", "msa_attn_bwd",
                  "msa_attn_fwd_blocksparse", "msa_decode_fwd_paged", "msa_append_kv_paged",
                  "msa_decode_fwd_noalloc"):
            getattr(L, f).restype = ctypes.c_int
        L.msa_status_string.argtypes = [ctypes.c_int]
        L.msa_status_string.restype = ctypes.c_char_p
        L.msa_last_error.argtypes = []
        L.msa_last_error.restype = ctypes.c_char_p
        L.msa_abi_version.argtypes = []
        L.msa_abi_version.restype = ctypes.c_int32
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != MSA_OK:
        L = lib()
        raise MsaError(status, f"{L.msa_status_string(status).decode()}: {L.msa_last_error().decode()}")


# ---------------------------------------------------------------- helpers

def _dtype_code(t) -> int:
    import torch
    if t == torch.float32:
        return MSA_DTYPE_F32
    if t == torch.bfloat16:
        return MSA_DTYPE_BF16
    raise TypeError(f"unsupported dtype {t}")


def _torch_dtype(code: int):
    import torch
    return torch.float32 if code == MSA_DTYPE_F32 else torch.bfloat16


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmsa must be contiguous")
    return t.data_ptr()


def _expect(t, name: str, shape=None, dtype=None, optional: bool = False) -> None:
    """Raise ValueError unless t has this shape and dtype and is contiguous."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_gpu(device, **tensors) -> None:
    """Raise ValueError unless every given tensor lives in GPU memory on
    `device`.  The library receives raw pointers: a tensor of the wrong size,
    type or device would otherwise become out-of-bounds device accesses."""
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be in GPU memory (it is on {t.device})")
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {device}")


def _expect_workspace(ws, need: int) -> None:
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace holds {ws.numel() * ws.element_size()} bytes, {need} needed")


def _expect_landmarks(Kbar, Vbar, B, Hkv, G, d, dtype) -> None:
    """Pooled landmarks [B][Hkv][G][d] in the input dtype (may be None when G = 0)."""
    _expect(Kbar, "Kbar", (B, Hkv, G, d), dtype, optional=G == 0)
    _expect(Vbar, "Vbar", (B, Hkv, G, d), dtype, optional=G == 0)


def _stream(t, stream) -> Optional[int]:
    import torch
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return torch.cuda.current_stream(t.device).cuda_stream


def attn_desc(batch, heads_q, heads_kv, seq_len, head_dim, window, num_landmarks, scale=None,
              in_dtype=MSA_DTYPE_BF16, out_dtype=None) -> AttnDesc:
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    if out_dtype is None:
        out_dtype = in_dtype
    return AttnDesc(batch, heads_q, heads_kv, seq_len, head_dim, window, num_landmarks, scale,
                    in_dtype, out_dtype)


def decode_desc(batch, heads_q, heads_kv, ctx_len, head_dim, window, num_landmarks, num_splits,
                scale=None, in_dtype=MSA_DTYPE_BF16, out_dtype=None, schedule=None) -> DecodeDesc:
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    if out_dtype is None:
        out_dtype = in_dtype
    return DecodeDesc(batch, heads_q, heads_kv, ctx_len, head_dim, window, num_landmarks, num_splits,
                      scale, in_dtype, out_dtype, _schedule_code(schedule))


# ---------------------------------------------------------------- compute

def msa_pool_landmarks(K, V, num_landmarks: int, Kbar=None, Vbar=None, stream=None):
    """Landmarks of K, V [B][Hkv][n][d]: (Kbar, Vbar) [B][Hkv][G][d]."""
    import torch
    B, Hkv, n, d = K.shape
    if V.shape != K.shape or V.dtype != K.dtype:
        raise ValueError("K and V must have the same shape and dtype")
    G = num_landmarks
    _expect(K, "K")
    _expect(V, "V")
    if Kbar is None:
        Kbar = torch.empty((B, Hkv, G, d), dtype=K.dtype, device=K.device)
    if Vbar is None:
        Vbar = torch.empty((B, Hkv, G, d), dtype=K.dtype, device=K.device)
    _expect_landmarks(Kbar, Vbar, B, Hkv, G, d, K.dtype)
    desc = attn_desc(B, Hkv, Hkv, n, d, 1, G, 1.0, _dtype_code(K.dtype))
    _on_gpu(K.device, K=K, V=V, Kbar=Kbar, Vbar=Vbar)
    _check(lib().msa_pool_landmarks(ctypes.byref(desc), _ptr(K), _ptr(V), _ptr(Kbar), _ptr(Vbar),
                                    _stream(K, stream)))
    return Kbar, Vbar


def msa_attn_fwd(Q, K, V, Kbar, Vbar, window: int, num_landmarks: int, scale: Optional[float] = None,
                 out_dtype=None, O=None, LSE=None, want_lse: bool = True, stream=None):
    """Window + landmark attention: (O [B][Hq][n][d], LSE [B][Hq][n] float32)."""
    import torch
    B, Hq, n, d = Q.shape
    Hkv = K.shape[1]
    if K.shape != (B, Hkv, n, d) or V.shape != K.shape:
        raise ValueError(f"K/V shape {tuple(K.shape)} does not match Q {tuple(Q.shape)}")
    if K.dtype != Q.dtype or V.dtype != Q.dtype:
        raise ValueError("Q, K, V must share a dtype")
    in_code = _dtype_code(Q.dtype)
    out_code = in_code if out_dtype is None else _dtype_code(out_dtype)
    dev = Q.device
    _expect(Q, "Q")
    _expect(K, "K")
    _expect(V, "V")
    _expect_landmarks(Kbar, Vbar, B, Hkv, num_landmarks, d, Q.dtype)
    if O is None:
        O = torch.empty((B, Hq, n, d), dtype=_torch_dtype(out_code), device=Q.device)
    if LSE is None and want_lse:
        LSE = torch.empty((B, Hq, n), dtype=torch.float32, device=Q.device)
    _expect(O, "O", (B, Hq, n, d), _torch_dtype(out_code))
    _expect(LSE, "LSE", (B, Hq, n), torch.float32, optional=True)
    desc = attn_desc(B, Hq, Hkv, n, d, window, num_landmarks, scale, in_code, out_code)
    _on_gpu(dev, Q=Q, K=K, V=V, Kbar=Kbar, Vbar=Vbar, O=O, LSE=LSE)
    _check(lib().msa_attn_fwd(ctypes.byref(desc), _ptr(Q), _ptr(K), _ptr(V), _ptr(Kbar), _ptr(Vbar),
                              _ptr(O), _ptr(LSE), _stream(Q, stream)))
    return O, LSE


def msa_attn_fwd_blocksparse(Q, K, V, block_counts, block_indices, causal: bool, scale: Optional[float] = None,
                             out_dtype=None, O=None, LSE=None, want_lse: bool = True, stream=None):
    """Attention over listed 64-key blocks per 128-row query block:
    block_counts int32 [B][Hq][T], block_indices int32 [B][Hq][T][max_blocks]
    (device tensors).  Returns (O, LSE)."""
    import torch
    B, Hq, n, d = Q.shape
    Hkv = K.shape[1]
    T = -(-n // LIST_QUERY_BLOCK)
    if K.shape != (B, Hkv, n, d) or V.shape != K.shape:
        raise ValueError("K/V shapes do not match Q")
    if block_counts.dtype != torch.int32 or tuple(block_counts.shape) != (B, Hq, T):
        raise ValueError(f"block_counts must be int32 [{B}][{Hq}][{T}]")
    if block_indices.dtype != torch.int32 or block_indices.dim() != 4 or \
            tuple(block_indices.shape[:3]) != (B, Hq, T):
        raise ValueError(f"block_indices must be int32 [{B}][{Hq}][{T}][max_blocks]")
    if K.dtype != Q.dtype or V.dtype != Q.dtype:
        raise ValueError("Q, K, V must share a dtype")
    in_code = _dtype_code(Q.dtype)
    out_code = in_code if out_dtype is None else _dtype_code(out_dtype)
    dev = Q.device
    _expect(Q, "Q")
    _expect(K, "K")
    _expect(V, "V")
    _expect(block_counts, "block_counts")
    _expect(block_indices, "block_indices")
    if O is None:
        O = torch.empty((B, Hq, n, d), dtype=_torch_dtype(out_code), device=Q.device)
    if LSE is None and want_lse:
        LSE = torch.empty((B, Hq, n), dtype=torch.float32, device=Q.device)
    _expect(O, "O", (B, Hq, n, d), _torch_dtype(out_code))
    _expect(LSE, "LSE", (B, Hq, n), torch.float32, optional=True)
    desc = attn_desc(B, Hq, Hkv, n, d, 1, 0, scale, in_code, out_code)
    _on_gpu(dev, Q=Q, K=K, V=V, block_counts=block_counts, block_indices=block_indices, O=O, LSE=LSE)
    _check(lib().msa_attn_fwd_blocksparse(ctypes.byref(desc), _ptr(block_counts), _ptr(block_indices),
                                          int(block_indices.shape[3]), 1 if causal else 0, _ptr(Q), _ptr(K),
                                          _ptr(V), _ptr(O), _ptr(LSE), _stream(Q, stream)))
    return O, LSE


def msa_attn_bwd_workspace_size(desc: AttnDesc) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().msa_attn_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(out)))
    return out.value


def msa_attn_bwd(Q, K, V, Kbar, Vbar, O, LSE, dO, window: int, num_landmarks: int,
                 scale: Optional[float] = None, out_dtype=None, workspace=None, dQ=None, dK=None, dV=None,
                 stream=None):
    """Gradients of msa_attn_fwd: (dQ [B][Hq][n][d], dK, dV [B][Hkv][n][d])
    for the upstream gradient dO, from the forward's O and LSE."""
    import torch
    B, Hq, n, d = Q.shape
    Hkv = K.shape[1]
    if K.shape != (B, Hkv, n, d) or V.shape != K.shape or O.shape != Q.shape or dO.shape != Q.shape:
        raise ValueError("shapes of K, V, O, dO do not match Q")
    if tuple(LSE.shape) != (B, Hq, n) or LSE.dtype != torch.float32:
        raise ValueError("LSE must be float32 [B][Hq][n]")
    if O.dtype != torch.bfloat16 or dO.dtype != torch.bfloat16:
        raise ValueError("O and dO must be bf16")
    if K.dtype != Q.dtype or V.dtype != Q.dtype:
        raise ValueError("Q, K, V must share a dtype")
    in_code = _dtype_code(Q.dtype)
    out_code = MSA_DTYPE_F32 if out_dtype is None else _dtype_code(out_dtype)
    dev = Q.device
    for t, name in ((Q, "Q"), (K, "K"), (V, "V"), (O, "O"), (LSE, "LSE"), (dO, "dO")):
        _expect(t, name)
    _expect_landmarks(Kbar, Vbar, B, Hkv, num_landmarks, d, Q.dtype)
    desc = attn_desc(B, Hq, Hkv, n, d, window, num_landmarks, scale, in_code, out_code)
    need = msa_attn_bwd_workspace_size(desc)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=Q.device)
    _expect_workspace(workspace, need)
    ws_bytes = workspace.numel() * workspace.element_size()
    odt = _torch_dtype(out_code)
    if dQ is None:
        dQ = torch.empty((B, Hq, n, d), dtype=odt, device=Q.device)
    if dK is None:
        dK = torch.empty((B, Hkv, n, d), dtype=odt, device=Q.device)
    if dV is None:
        dV = torch.empty((B, Hkv, n, d), dtype=odt, device=Q.device)
    _expect(dQ, "dQ", (B, Hq, n, d), odt)
    _expect(dK, "dK", (B, Hkv, n, d), odt)
    _expect(dV, "dV", (B, Hkv, n, d), odt)
    _on_gpu(dev, Q=Q, K=K, V=V, Kbar=Kbar, Vbar=Vbar, O=O, LSE=LSE, dO=dO, workspace=workspace, dQ=dQ, dK=dK,
            dV=dV)
    _check(lib().msa_attn_bwd(ctypes.byref(desc), _ptr(Q), _ptr(K), _ptr(V), _ptr(Kbar), _ptr(Vbar), _ptr(O),
                              _ptr(LSE), _ptr(dO), _ptr(workspace), ws_bytes, _ptr(dQ), _ptr(dK), _ptr(dV),
                              _stream(Q, stream)))
    return dQ, dK, dV


def msa_decode_workspace_size(desc: DecodeDesc) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().msa_decode_workspace_size(ctypes.byref(desc), ctypes.byref(out)))
    return out.value


def msa_decode_fwd(q, Kc, Vc, Kbar, Vbar, window: int, num_landmarks: int, num_splits: int,
                   scale: Optional[float] = None, out_dtype=None, workspace=None, O=None, LSE=None,
                   want_lse: bool = True, stream=None, schedule=None):
    """Decode for the query at position ctx-1: (O [B][Hq][d], LSE [B][Hq]).
    ``workspace`` (uint8 or float32 device tensor) receives the per-chunk
    partials; it is allocated here when not given."""
    import torch
    B, Hq, d = q.shape
    Hkv, ctx = Kc.shape[1], Kc.shape[2]
    if Kc.shape != (B, Hkv, ctx, d) or Vc.shape != Kc.shape:
        raise ValueError("cache shapes do not match q")
    if Kc.dtype != q.dtype or Vc.dtype != q.dtype:
        raise ValueError("q and the caches must share a dtype")
    in_code = _dtype_code(q.dtype)
    out_code = in_code if out_dtype is None else _dtype_code(out_dtype)
    dev = q.device
    _expect(q, "q")
    _expect(Kc, "Kc")
    _expect(Vc, "Vc")
    _expect_landmarks(Kbar, Vbar, B, Hkv, num_landmarks, d, q.dtype)
    desc = decode_desc(B, Hq, Hkv, ctx, d, window, num_landmarks, num_splits, scale, in_code, out_code, schedule)
    need = msa_decode_workspace_size(desc)
    if workspace is None:
        workspace = torch.empty(max(need // 4, 1), dtype=torch.float32, device=q.device)
    _expect_workspace(workspace, need)
    ws_bytes = workspace.numel() * workspace.element_size()
    if O is None:
        O = torch.empty((B, Hq, d), dtype=_torch_dtype(out_code), device=q.device)
    if LSE is None and want_lse:
        LSE = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _expect(O, "O", (B, Hq, d), _torch_dtype(out_code))
    _expect(LSE, "LSE", (B, Hq), torch.float32, optional=True)
    _on_gpu(dev, q=q, Kc=Kc, Vc=Vc, Kbar=Kbar, Vbar=Vbar, workspace=workspace, O=O, LSE=LSE)
    _check(lib().msa_decode_fwd(ctypes.byref(desc), _ptr(q), _ptr(Kc), _ptr(Vc), _ptr(Kbar), _ptr(Vbar),
                                _ptr(workspace), ws_bytes, _ptr(O), _ptr(LSE), _stream(q, stream)))
    return O, LSE


NOALLOC_SCRATCH_BYTES = 32 << 20


def msa_decode_fwd_noalloc(q, Kc, Vc, Kbar, Vbar, window: int, num_landmarks: int, num_splits: int,
                           scale: Optional[float] = None, O=None, LSE=None, stream=None, schedule=None):
    """msa_decode_fwd without a workspace: the split schedule's partials live
    in the library's own device array (NOALLOC_SCRATCH_BYTES per GPU).  For
    callers that cannot allocate, pass O (and LSE); the library allocates
    nothing.  Overlapping calls on one GPU race on that array."""
    import torch
    B, Hq, d = q.shape
    Hkv, ctx = Kc.shape[1], Kc.shape[2]
    if Kc.shape != (B, Hkv, ctx, d) or Vc.shape != Kc.shape:
        raise ValueError("cache shapes do not match q")
    if Kc.dtype != q.dtype or Vc.dtype != q.dtype:
        raise ValueError("q and the caches must share a dtype")
    in_code = _dtype_code(q.dtype)
    if O is None:
        O = torch.empty((B, Hq, d), dtype=q.dtype, device=q.device)
    out_code = _dtype_code(O.dtype)
    dev = q.device
    _expect(q, "q")
    _expect(Kc, "Kc")
    _expect(Vc, "Vc")
    _expect_landmarks(Kbar, Vbar, B, Hkv, num_landmarks, d, q.dtype)
    _expect(O, "O", (B, Hq, d), _torch_dtype(out_code))
    _expect(LSE, "LSE", (B, Hq), torch.float32, optional=True)
    desc = decode_desc(B, Hq, Hkv, ctx, d, window, num_landmarks, num_splits, scale, in_code, out_code, schedule)
    _on_gpu(dev, q=q, Kc=Kc, Vc=Vc, Kbar=Kbar, Vbar=Vbar, O=O, LSE=LSE)
    _check(lib().msa_decode_fwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(Kc), _ptr(Vc), _ptr(Kbar), _ptr(Vbar),
                                        _ptr(O), _ptr(LSE), _stream(q, stream)))
    return O, LSE


def msa_decode_fwd_varlen(q, Kc, Vc, Kbar, Vbar, ctx_lens, window: int, num_landmarks: int,
                          num_splits: int, scale: Optional[float] = None, out_dtype=None, workspace=None,
                          O=None, LSE=None, want_lse: bool = True, stream=None, schedule=None):
    """Decode of sequences of different lengths: sequence b holds
    ctx_lens[b] tokens (int32 device tensor [B]) of a cache with capacity
    Kc.shape[2] rows; its query is at position ctx_lens[b]-1.  Landmark
    blocks have length capacity / num_landmarks.  (O [B][Hq][d], LSE [B][Hq])."""
    import torch
    B, Hq, d = q.shape
    Hkv, cap = Kc.shape[1], Kc.shape[2]
    if Kc.shape != (B, Hkv, cap, d) or Vc.shape != Kc.shape:
        raise ValueError("cache shapes do not match q")
    if ctx_lens.dtype != torch.int32 or tuple(ctx_lens.shape) != (B,):
        raise ValueError("ctx_lens must be an int32 tensor of shape [B]")
    if Kc.dtype != q.dtype or Vc.dtype != q.dtype:
        raise ValueError("q and the caches must share a dtype")
    in_code = _dtype_code(q.dtype)
    out_code = in_code if out_dtype is None else _dtype_code(out_dtype)
    dev = q.device
    _expect(q, "q")
    _expect(Kc, "Kc")
    _expect(Vc, "Vc")
    _expect(ctx_lens, "ctx_lens")
    _expect_landmarks(Kbar, Vbar, B, Hkv, num_landmarks, d, q.dtype)
    desc = decode_desc(B, Hq, Hkv, cap, d, window, num_landmarks, num_splits, scale, in_code, out_code, schedule)
    need = msa_decode_workspace_size(desc)
    if workspace is None:
        workspace = torch.empty(max(need // 4, 1), dtype=torch.float32, device=q.device)
    _expect_workspace(workspace, need)
    ws_bytes = workspace.numel() * workspace.element_size()
    if O is None:
        O = torch.empty((B, Hq, d), dtype=_torch_dtype(out_code), device=q.device)
    if LSE is None and want_lse:
        LSE = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _expect(O, "O", (B, Hq, d), _torch_dtype(out_code))
    _expect(LSE, "LSE", (B, Hq), torch.float32, optional=True)
    _on_gpu(dev, q=q, Kc=Kc, Vc=Vc, ctx_lens=ctx_lens, Kbar=Kbar, Vbar=Vbar, workspace=workspace, O=O, LSE=LSE)
    _check(lib().msa_decode_fwd_varlen(ctypes.byref(desc), _ptr(ctx_lens), _ptr(q), _ptr(Kc), _ptr(Vc),
                                       _ptr(Kbar), _ptr(Vbar), _ptr(workspace), ws_bytes, _ptr(O), _ptr(LSE),
                                       _stream(q, stream)))
    return O, LSE


def msa_append_kv(k_new, v_new, positions, Kc, Vc, Kbar, Vbar, num_landmarks: int, stream=None):
    """Store one token per sequence (k_new, v_new [B][Hkv][d]) at row
    positions[b] (int32 device tensor [B]; outside [0, capacity) = skip) of
    the caches, in place, and re-pool the landmark block that row completes."""
    import torch
    B, Hkv, cap, d = Kc.shape
    if Vc.shape != Kc.shape or tuple(k_new.shape) != (B, Hkv, d) or v_new.shape != k_new.shape:
        raise ValueError("k_new/v_new [B][Hkv][d] must match the caches [B][Hkv][C][d]")
    if positions.dtype != torch.int32 or tuple(positions.shape) != (B,):
        raise ValueError("positions must be an int32 tensor of shape [B]")
    if k_new.dtype != Kc.dtype or v_new.dtype != Kc.dtype or Vc.dtype != Kc.dtype:
        raise ValueError("new rows and caches must share a dtype")
    dev = Kc.device
    _expect(Kc, "Kc")
    for t, name in ((Vc, "Vc"), (k_new, "k_new"), (v_new, "v_new"), (positions, "positions")):
        _expect(t, name)
    _expect_landmarks(Kbar, Vbar, B, Hkv, num_landmarks, d, Kc.dtype)
    desc = decode_desc(B, Hkv, Hkv, cap, d, 1, num_landmarks, 1, 1.0, _dtype_code(Kc.dtype))
    _on_gpu(dev, Kc=Kc, Vc=Vc, k_new=k_new, v_new=v_new, positions=positions, Kbar=Kbar, Vbar=Vbar)
    _check(lib().msa_append_kv(ctypes.byref(desc), _ptr(positions), _ptr(k_new), _ptr(v_new), _ptr(Kc),
                               _ptr(Vc), _ptr(Kbar), _ptr(Vbar), _stream(Kc, stream)))


def msa_decode_fwd_paged(q, Kpages, Vpages, block_table, Kbar, Vbar, ctx_lens, window: int, num_landmarks: int,
                         num_splits: int, scale: Optional[float] = None, out_dtype=None, workspace=None, O=None,
                         LSE=None, want_lse: bool = True, stream=None, schedule=None):
    """Decode over paged caches: pools [num_pages][Hkv][page][d], block_table
    int32 [B][pages per sequence] (capacity = pages per sequence x page)."""
    import torch
    B, Hq, d = q.shape
    num_pages, Hkv, page, _ = Kpages.shape
    if Vpages.shape != Kpages.shape or Kpages.shape[3] != d:
        raise ValueError("page pools must be [num_pages][Hkv][page][d] and match q")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B][pages per sequence]")
    if ctx_lens.dtype != torch.int32 or tuple(ctx_lens.shape) != (B,):
        raise ValueError("ctx_lens must be an int32 tensor of shape [B]")
    cap = block_table.shape[1] * page
    if cap >= 1 << 31:
        raise ValueError(f"capacity {cap} (pages per sequence x page) must be < 2^31 rows")
    if Kpages.dtype != q.dtype or Vpages.dtype != q.dtype:
        raise ValueError("q and the page pools must share a dtype")
    in_code = _dtype_code(q.dtype)
    out_code = in_code if out_dtype is None else _dtype_code(out_dtype)
    dev = q.device
    _expect(q, "q")
    for t, name in ((Kpages, "Kpages"), (Vpages, "Vpages"), (block_table, "block_table"), (ctx_lens, "ctx_lens")):
        _expect(t, name)
    _expect_landmarks(Kbar, Vbar, B, Hkv, num_landmarks, d, q.dtype)
    desc = decode_desc(B, Hq, Hkv, cap, d, window, num_landmarks, num_splits, scale, in_code, out_code, schedule)
    need = msa_decode_workspace_size(desc)
    if workspace is None:
        workspace = torch.empty(max(need // 4, 1), dtype=torch.float32, device=q.device)
    _expect_workspace(workspace, need)
    ws_bytes = workspace.numel() * workspace.element_size()
    if O is None:
        O = torch.empty((B, Hq, d), dtype=_torch_dtype(out_code), device=q.device)
    if LSE is None and want_lse:
        LSE = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _expect(O, "O", (B, Hq, d), _torch_dtype(out_code))
    _expect(LSE, "LSE", (B, Hq), torch.float32, optional=True)
    _on_gpu(dev, q=q, Kpages=Kpages, Vpages=Vpages, block_table=block_table, ctx_lens=ctx_lens, Kbar=Kbar,
            Vbar=Vbar, workspace=workspace, O=O, LSE=LSE)
    _check(lib().msa_decode_fwd_paged(ctypes.byref(desc), page, num_pages, _ptr(block_table), _ptr(ctx_lens),
                                      _ptr(q), _ptr(Kpages), _ptr(Vpages), _ptr(Kbar), _ptr(Vbar), _ptr(workspace),
                                      ws_bytes, _ptr(O), _ptr(LSE), _stream(q, stream)))
    return O, LSE


def msa_append_kv_paged(k_new, v_new, positions, Kpages, Vpages, block_table, Kbar, Vbar, num_landmarks: int,
                        stream=None):
    """msa_append_kv over paged caches (see msa_decode_fwd_paged)."""
    import torch
    num_pages, Hkv, page, d = Kpages.shape
    B = block_table.shape[0]
    if Vpages.shape != Kpages.shape or tuple(k_new.shape) != (B, Hkv, d) or v_new.shape != k_new.shape:
        raise ValueError("k_new/v_new [B][Hkv][d] must match the page pools")
    if positions.dtype != torch.int32 or tuple(positions.shape) != (B,):
        raise ValueError("positions must be an int32 tensor of shape [B]")
    if block_table.dtype != torch.int32 or block_table.dim() != 2:
        raise ValueError("block_table must be int32 [B][pages per sequence]")
    cap = block_table.shape[1] * page
    if cap >= 1 << 31:
        raise ValueError(f"capacity {cap} (pages per sequence x page) must be < 2^31 rows")
    if k_new.dtype != Kpages.dtype or v_new.dtype != Kpages.dtype or Vpages.dtype != Kpages.dtype:
        raise ValueError("new rows and page pools must share a dtype")
    dev = Kpages.device
    _expect(Kpages, "Kpages")
    for t, name in ((Vpages, "Vpages"), (block_table, "block_table"), (positions, "positions"),
                    (k_new, "k_new"), (v_new, "v_new")):
        _expect(t, name)
    _expect_landmarks(Kbar, Vbar, B, Hkv, num_landmarks, d, Kpages.dtype)
    desc = decode_desc(B, Hkv, Hkv, cap, d, 1, num_landmarks, 1, 1.0, _dtype_code(Kpages.dtype))
    _on_gpu(dev, Kpages=Kpages, Vpages=Vpages, block_table=block_table, positions=positions, k_new=k_new,
            v_new=v_new, Kbar=Kbar, Vbar=Vbar)
    _check(lib().msa_append_kv_paged(ctypes.byref(desc), page, num_pages, _ptr(block_table), _ptr(positions),
                                     _ptr(k_new), _ptr(v_new), _ptr(Kpages), _ptr(Vpages), _ptr(Kbar), _ptr(Vbar),
                                     _stream(Kpages, stream)))


def decode_partials(workspace, num_splits: int, batch: int, heads_q: int, head_dim: int):
    """Views of the per-chunk results held in a decode workspace:
    (o [S][B][Hq][d], lse [S][B][Hq]), both float32."""
    ws = workspace.view(-1).view(dtype=__import__("torch").float32)
    n_o = num_splits * batch * heads_q * head_dim
    o = ws[:n_o].view(num_splits, batch, heads_q, head_dim)
    lse = ws[n_o:n_o + num_splits * batch * heads_q].view(num_splits, batch, heads_q)
    return o, lse


# ---------------------------------------------------------------- host-only plan queries

def msa_plan_rows(desc: AttnDesc) -> Tuple[np.ndarray, np.ndarray]:
    n = desc.seq_len
    win_lo = np.zeros(max(n, 1), dtype=np.int32)
    lm = np.zeros(max(n, 1), dtype=np.int32)
    _check(lib().msa_plan_rows(ctypes.byref(desc), win_lo.ctypes.data, lm.ctypes.data))
    return win_lo[:n], lm[:n]


def msa_plan_tiles(desc: AttnDesc):
    """(tiles int32 [count, 4] = (query_tile, kind, tile, interior), bm, bn)."""
    cnt = ctypes.c_int64(0)
    bm = ctypes.c_int32(0)
    bn = ctypes.c_int32(0)
    _check(lib().msa_plan_tiles(ctypes.byref(desc), None, 0, ctypes.byref(cnt), ctypes.byref(bm),
                                ctypes.byref(bn)))
    out = np.zeros((max(cnt.value, 1), 4), dtype=np.int32)
    _check(lib().msa_plan_tiles(ctypes.byref(desc), out.ctypes.data, cnt.value, ctypes.byref(cnt),
                                ctypes.byref(bm), ctypes.byref(bn)))
    return out[:cnt.value], bm.value, bn.value


def msa_plan_decode(desc: DecodeDesc):
    """(chunk_bounds int32 [S+1], visible landmarks, entries)."""
    bounds = np.zeros(desc.num_splits + 1, dtype=np.int32)
    lm = ctypes.c_int32(0)
    ent = ctypes.c_int32(0)
    _check(lib().msa_plan_decode(ctypes.byref(desc), bounds.ctypes.data, ctypes.byref(lm), ctypes.byref(ent)))
    return bounds, lm.value, ent.value


def msa_plan_decode_varlen(desc: DecodeDesc, ctx: int):
    """Plan of one sequence of ctx tokens in a cache of capacity
    desc.ctx_len: (chunk_bounds int32 [S+1], visible landmarks, entries)."""
    bounds = np.zeros(desc.num_splits + 1, dtype=np.int32)
    lm = ctypes.c_int32(0)
    ent = ctypes.c_int32(0)
    _check(lib().msa_plan_decode_varlen(ctypes.byref(desc), int(ctx), bounds.ctypes.data, ctypes.byref(lm),
                                        ctypes.byref(ent)))
    return bounds, lm.value, ent.value


def abi_version() -> int:
    return lib().msa_abi_version()
