"""Seeded synthetic workloads for window + landmark sparse attention.

This module holds shapes and random-number recipes only.  It computes no step
of the attention method itself, so that both the fp64 oracle (``oracle/``) and
the HIP path (``long_context_sparse_msa_amd``) can be fed identical inputs
without sharing any arithmetic.

Shapes follow the workloads described on the pages:
  * "Scaling GPU Cluster for Million Token Context", sections "Why Sparse
    Attention Changes the Game" and "A Concrete Example: Configuring for 1M
    Token Inference": window 4096, 512 landmark ("global") tokens, sequence
    length 2**20.
  * "Training at 1M+ Token Context: Ring Attention, YaRN, NTK-Aware Scaling
    GPU Cost", the memory paragraph: 64 query heads sharing 8 KV heads of
    head dimension 128 (a 70B-like model).
The pages measure on long-document benchmarks that are not available here;
N(0, 1) tensors of the same shapes stand in for them.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Prefill:
    name: str
    batch: int
    heads_q: int
    heads_kv: int
    seq_len: int
    head_dim: int
    window: int
    num_landmarks: int
    dtype: str            # "f32" or "bf16": input dtype of Q, K, V
    out_dtype: str        # dtype of O
    peaky: bool = False   # 1% of key rows scaled by 8 (see ``peaky_rows``)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


@dataclasses.dataclass(frozen=True)
class Decode:
    name: str
    batch: int
    heads_q: int
    heads_kv: int
    ctx_len: int
    head_dim: int
    window: int
    num_landmarks: int
    num_splits: int
    dtype: str = "bf16"

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


# The five workloads.  Sizes are those of the window/landmark pattern on the
# pages; the first is small enough for the fp64 oracle to check every row.
TINY_FP32 = Prefill("tiny_fp32", 1, 2, 2, 2048, 64, 256, 16, "f32", "f32")
BF16_32K = Prefill("bf16_32k", 1, 8, 8, 32768, 128, 4096, 512, "bf16", "bf16")
BF16_32K_PEAKY = dataclasses.replace(BF16_32K, name="bf16_32k_peaky", peaky=True)
GQA_128K = Prefill("gqa_128k", 1, 64, 8, 131072, 128, 4096, 512, "bf16", "bf16")
GQA_1M = Prefill("gqa_1m", 1, 64, 8, 1048576, 128, 4096, 512, "bf16", "bf16")
DECODE_512K = Decode("decode_512k", 64, 64, 8, 524288, 128, 4096, 512, 16)

PREFILL_WORKLOADS = {c.name: c for c in (TINY_FP32, BF16_32K, BF16_32K_PEAKY, GQA_128K, GQA_1M)}

# Seeds: seed 0 for the plain N(0,1) draw, seed 1 for the peaky variant.
SEED_PLAIN = 0
SEED_PEAKY = 1


def host_normal(shape, seed: int, stream: int = 0) -> np.ndarray:
    """float32 N(0,1) tensor from numpy's PCG64, seeded by (seed, stream)."""
    rng = np.random.default_rng([seed, stream])
    return rng.standard_normal(size=shape, dtype=np.float32)


def peaky_rows(n: int, seed: int, batch: int, heads_kv: int) -> np.ndarray:
    """Positions whose K rows get multiplied by 8: n//100 distinct rows per
    (batch, KV head), drawn without replacement from a seeded generator.
    Returns int64 [batch, heads_kv, n//100], each row sorted."""
    rng = np.random.default_rng([seed, 99])
    cnt = n // 100
    out = np.empty((batch, heads_kv, cnt), dtype=np.int64)
    for b in range(batch):
        for g in range(heads_kv):
            out[b, g] = np.sort(rng.choice(n, size=cnt, replace=False))
    return out


def host_prefill_inputs(cfg: Prefill, seed: Optional[int] = None):
    """Q, K, V as float32 numpy arrays [B][H][n][d] (values already rounded
    to bf16 when cfg.dtype == "bf16", so that host and device see the same
    numbers).  Intended for sizes that fit comfortably in host memory."""
    import torch

    if seed is None:
        seed = SEED_PEAKY if cfg.peaky else SEED_PLAIN
    B, Hq, Hkv, n, d = cfg.batch, cfg.heads_q, cfg.heads_kv, cfg.seq_len, cfg.head_dim
    q = host_normal((B, Hq, n, d), seed, 0)
    k = host_normal((B, Hkv, n, d), seed, 1)
    v = host_normal((B, Hkv, n, d), seed, 2)
    if cfg.peaky:
        rows = peaky_rows(n, seed, B, Hkv)
        for b in range(B):
            for g in range(Hkv):
                k[b, g, rows[b, g]] *= 8.0
    if cfg.dtype == "bf16":
        q, k, v = (torch.from_numpy(x).to(torch.bfloat16).float().numpy() for x in (q, k, v))
    return q, k, v


def device_normal(shape, seed: int, stream: int, dtype, device):
    """N(0,1) tensor generated on ``device`` by torch's Philox generator
    seeded with seed*1000+stream, drawn in float32 and rounded to ``dtype``
    (round-to-nearest-even for bf16).  Large tensors are filled in slabs so no
    float32 copy of the whole tensor is ever held."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000 + stream)
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    slab = 1 << 28
    for s in range(0, flat.numel(), slab):
        e = min(flat.numel(), s + slab)
        flat[s:e] = torch.randn(e - s, generator=g, dtype=torch.float32, device=device).to(dtype)
    return out


def device_prefill_inputs(cfg: Prefill, device, seed: Optional[int] = None):
    """Q, K, V on ``device`` in the workload's dtype, layout [B][H][n][d]."""
    import torch

    if seed is None:
        seed = SEED_PEAKY if cfg.peaky else SEED_PLAIN
    dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    B, Hq, Hkv, n, d = cfg.batch, cfg.heads_q, cfg.heads_kv, cfg.seq_len, cfg.head_dim
    q = device_normal((B, Hq, n, d), seed, 0, dt, device)
    k = device_normal((B, Hkv, n, d), seed, 1, dt, device)
    v = device_normal((B, Hkv, n, d), seed, 2, dt, device)
    if cfg.peaky:
        rows = torch.from_numpy(peaky_rows(n, seed, B, Hkv)).to(device)
        for b in range(B):
            for g in range(Hkv):
                k[b, g, rows[b, g]] *= 8
    return q, k, v


def device_decode_inputs(cfg: Decode, device, seed: int = SEED_PLAIN):
    """q [B][Hq][d], K/V caches [B][Hkv][ctx][d] on ``device``."""
    import torch

    dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    B, Hq, Hkv, ctx, d = cfg.batch, cfg.heads_q, cfg.heads_kv, cfg.ctx_len, cfg.head_dim
    q = device_normal((B, Hq, d), seed, 10, dt, device)
    kc = device_normal((B, Hkv, ctx, d), seed, 11, dt, device)
    vc = device_normal((B, Hkv, ctx, d), seed, 12, dt, device)
    return q, kc, vc


def decode_lengths(batch: int, capacity: int, seed: int = SEED_PLAIN, lo_frac: float = 0.5) -> np.ndarray:
    """Seeded per-sequence context lengths for incremental decode: uniform
    integers in [lo_frac * capacity, capacity] (a batch of long documents at
    different points of their generation).  int32 [batch]."""
    rng = np.random.default_rng(1000 + seed)
    lo = max(1, int(lo_frac * capacity))
    return rng.integers(lo, capacity + 1, size=batch).astype(np.int32)


def band_block_lists(batch: int, heads: int, n: int, blocks: int = 16, block_tokens: int = 128,
                     query_block: int = 128, key_block: int = 64):
    """Block lists of the pattern in which each 128-token block attends to 16
    blocks around it, half to the left and half to the right ("Million Token
    Context Window Optimization: What Actually Works", indexing section):
    query block t lists the 128-token blocks t - blocks/2 .. t + blocks/2 - 1
    (clipped to the sequence), written as key_block-sized indices.  Returns
    (counts int32 [B][H][T], indices int32 [B][H][T][max_blocks])."""
    T = -(-n // query_block)
    per = block_tokens // key_block
    nkb = -(-n // key_block)
    maxb = blocks * per
    counts = np.zeros((batch, heads, T), np.int32)
    idx = np.full((batch, heads, T, maxb), -1, np.int32)
    for t in range(T):
        c0 = t * query_block // block_tokens
        kbs = [kb for c in range(c0 - blocks // 2, c0 + blocks // 2) if c >= 0
               for kb in range(c * per, (c + 1) * per) if kb < nkb]
        counts[:, :, t] = len(kbs)
        idx[:, :, t, :len(kbs)] = kbs
    return counts, idx


def global_local_block_lists(batch: int, heads: int, n: int, global_blocks: int = 2, local_blocks: int = 16,
                             block_tokens: int = 128, query_block: int = 128, key_block: int = 64):
    """Block lists of the global + local pattern: global tokens that attend
    to every token and that every token attends to, plus a local sliding
    window ("Training at 1M+ Token Context: Ring Attention, YaRN, NTK-Aware
    Scaling GPU Cost", Block-Sparse Flash Attention paragraph), at block
    granularity and without a causal mask.  The first `global_blocks`
    128-token blocks are the global tokens: their query blocks list every
    key block; every other query block t lists the global blocks and the
    128-token blocks t - local_blocks/2 .. t + local_blocks/2 - 1 (clipped,
    each block once), as key_block-sized indices in ascending order.
    Returns (counts int32 [B][H][T], indices int32 [B][H][T][max_blocks])."""
    T = -(-n // query_block)
    per = block_tokens // key_block
    nkb = -(-n // key_block)
    nblk = -(-n // block_tokens)
    counts = np.zeros((batch, heads, T), np.int32)
    idx = np.full((batch, heads, T, nkb), -1, np.int32)
    for t in range(T):
        c0 = t * query_block // block_tokens
        if c0 < global_blocks:
            blks = list(range(nblk))
        else:
            blks = sorted(set(range(min(global_blocks, nblk))) |
                          {c for c in range(c0 - local_blocks // 2, c0 + local_blocks // 2) if 0 <= c < nblk})
        kbs = [kb for c in blks for kb in range(c * per, (c + 1) * per) if kb < nkb]
        counts[:, :, t] = len(kbs)
        idx[:, :, t, :len(kbs)] = kbs
    return counts, idx


def random_block_lists(batch: int, heads: int, n: int, max_blocks: int, seed: int,
                       query_block: int = 128, key_block: int = 64):
    """Seeded random lists for tests: counts uniform in [0, max_blocks],
    indices uniform in [-2, nkb + 2) (so some are out of range), repeats
    allowed."""
    rng = np.random.default_rng(2000 + seed)
    T = -(-n // query_block)
    nkb = -(-n // key_block)
    counts = rng.integers(0, max_blocks + 1, size=(batch, heads, T)).astype(np.int32)
    idx = rng.integers(-2, nkb + 2, size=(batch, heads, T, max_blocks)).astype(np.int32)
    return counts, idx


def sample_rows(n: int, head: int, count: int = 4096, window: int = 0, block: int = 0) -> np.ndarray:
    """Seeded sample of query rows for one head (generator seeded 12345+head),
    plus forced edge rows around the start, the window edge, the first
    landmark boundaries and the end of the sequence.  Sorted, unique."""
    rng = np.random.default_rng(12345 + head)
    take = min(count, n)
    rows = rng.choice(n, size=take, replace=False)
    forced = [0, 1, 2, n - 2, n - 1]
    if window:
        forced += [window - 2, window - 1, window]
        if block:
            forced += [window - 1 + block, window - 2 + block, window - 1 + 2 * block]
    forced = [r for r in forced if 0 <= r < n]
    return np.unique(np.concatenate([rows, np.array(forced, dtype=rows.dtype)]))
