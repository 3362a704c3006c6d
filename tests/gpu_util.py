"""Helpers for the GPU parity tests: device selection, bf16 rounding on the
host, oracle comparisons on sampled rows, and the tolerances.

Tolerances (the bounds of the window + landmark attention specification):
  float32 inputs : max |dO| <= 1e-5, max |dLSE| <= 1e-5
  bf16 inputs    : max |dO| <= 1e-2, mean |dO| <= 1e-3, max |dLSE| <= 1e-3
graded on the kernel's float32 epilogue (same kernel, float32 output); the
bf16 store is then checked to be exactly round-to-nearest-even of it.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import msa_oracle as orc

TOL_F32 = dict(max_o=1e-5, mean_o=1e-5, max_lse=1e-5)
TOL_BF16 = dict(max_o=1e-2, mean_o=1e-3, max_lse=1e-3)


def dev():
    return torch.device("cuda:0")


def host64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a device tensor (bf16 and f32 widen exactly)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_close(o_gpu, lse_gpu, o_ref, lse_ref, tol, what=""):
    do = np.abs(np.asarray(o_gpu, np.float64) - o_ref)
    dl = np.abs(np.asarray(lse_gpu, np.float64) - lse_ref)
    stats = dict(max_o=float(do.max()), mean_o=float(do.mean()), max_lse=float(dl.max()))
    print(f"[parity] {what}: max|dO|={stats['max_o']:.3e} mean|dO|={stats['mean_o']:.3e} "
          f"max|dLSE|={stats['max_lse']:.3e}", flush=True)
    assert stats["max_o"] <= tol["max_o"], (what, stats)
    assert stats["mean_o"] <= tol["mean_o"], (what, stats)
    assert stats["max_lse"] <= tol["max_lse"], (what, stats)
    return stats


def check_rows(Q, K, V, O32, LSE, w, G, scale, rows_by_head, tol, what, group_span=512, O16=None):
    """Compare GPU rows against the oracle on the given rows of each head.
    Q, K, V, O32, LSE are device tensors; K/V are copied per KV head.
    With O16 (the bf16 store of the same run), also grade the shipped bf16
    output: each element must lie within the float32 bound plus half a bf16
    ulp of its float32 value (a correctly rounded store adds at most that,
    2^-6 where |O| >= 4), and its raw distance to the oracle is printed."""
    B, Hq, n, d = Q.shape
    Hkv = K.shape[1]
    grp = Hq // Hkv
    worst = dict(max_o=0.0, mean_o=0.0, max_lse=0.0)
    raw = dict(max=0.0, sum=0.0, count=0, big_over=0, big=0)
    for g in range(Hkv):
        heads = [h for h in range(g * grp, (g + 1) * grp) if h in rows_by_head]
        if not heads:
            continue
        Kh = host64(K[:, g:g + 1])
        Vh = host64(V[:, g:g + 1])
        Kb = orc.pool(Kh, G) if G else None
        Vb = orc.pool(Vh, G) if G else None
        for h in heads:
            rows = np.asarray(rows_by_head[h], dtype=np.int64)
            ridx = torch.from_numpy(rows).to(Q.device)
            Qr = np.zeros((B, 1, n, d))  # only the sampled rows are touched
            Qr[:, 0, rows] = host64(Q[:, h].index_select(1, ridx))
            res = orc.attn(Qr, Kh, Vh, w, G, scale, rows={0: rows}, Kbar=Kb, Vbar=Vb,
                           group_span=group_span)
            _, o_ref, lse_ref = res[0]
            o_gpu = host64(O32[:, h].index_select(1, ridx))
            l_gpu = host64(LSE[:, h].index_select(1, ridx))
            s = assert_close(o_gpu, l_gpu, o_ref, lse_ref, tol, f"{what} head {h} ({len(rows)} rows)")
            for k in worst:
                worst[k] = max(worst[k], s[k])
            if O16 is not None:
                d16 = np.abs(host64(O16[:, h].index_select(1, ridx)) - o_ref)
                bound = tol["max_o"] + bf16_half_ulp(o_gpu)
                over = d16 > bound
                assert not over.any(), (f"{what} head {h}: bf16 output off by {d16[over].max():.3e}, "
                                        f"beyond max|dO| + half a bf16 ulp at {int(over.sum())} elements")
                big = np.abs(o_ref) >= 4
                raw["max"] = max(raw["max"], float(d16.max()))
                raw["sum"] += float(d16.sum())
                raw["count"] += d16.size
                raw["big"] += int(big.sum())
                raw["big_over"] += int((d16[big] > 1e-2).sum())
    if O16 is not None and raw["count"]:
        print(f"[info] {what}: bf16 store vs oracle max {raw['max']:.3e} mean {raw['sum'] / raw['count']:.3e}; "
              f"{raw['big']} elements with |O| >= 4, {raw['big_over']} of them off by > 1e-2", flush=True)
    return worst


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half the spacing of bf16 values (8 significant bits) in the binade of
    each |x|: the largest error of round-to-nearest into bf16."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return np.ldexp(1.0, (e - 8).astype(np.int64))


def bf16_rne(x: torch.Tensor) -> torch.Tensor:
    """Round float32 to bf16 with round-to-nearest-even (torch's cast)."""
    return x.to(torch.bfloat16)
