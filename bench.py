#!/usr/bin/env python3
"""Benchmark of the window + landmark sparse-attention hot path on one MI355X.

One step is one pass over every stage of the path on synthetic inputs that
are already resident in HBM:
  1. landmark pooling of K and V (128K-token GQA workload),
  2. sparse-attention prefill of that workload (64 query / 8 KV heads,
     d = 128, window 4096, 512 landmarks), O in bf16 and LSE in float32,
  3. split-KV decode (16 chunks + LSE merge) for 64 sequences with a
     512K-token bf16 cache (landmarks of the cache pooled once at set-up,
     timed separately).
`value` is the prefill's useful TFLOP/s (4*d FLOPs per visible
(query, key-or-landmark) pair, pooling included in the time); decode is
reported as algorithmic HBM GB/s alongside.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-attn fwd TFLOP/s + MFMA util at n=128K; decode HBM GB/s at 512K ctx"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def kernel_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "long_context_sparse_msa_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(name, src_files, per_launch_scale=1.0):
    """HBM bytes per launch measured with rocprofv3 counters (FETCH_SIZE +
    WRITE_SIZE, scaled by the copy-kernel calibration), if they were taken
    on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_hash(*src_files):
        return None
    return rec.get("bytes_per_launch")


COPY_BYTES = 1 << 30


def _pmc_rows(path, counter):
    import csv

    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                out[r["Dispatch_Id"]] = (r["Kernel_Name"], float(r["Counter_Value"]))
    return out


def summarize_pmc(fetch_csv, write_csv):
    """HBM bytes per launch of the prefill and decode kernels from a
    rocprofv3 --pmc run of this bench with --calibrate-copy.  Each counter
    (KiB per dispatch) is scaled by what it reads for the 1 GiB copy."""
    fetch = _pmc_rows(fetch_csv, "FETCH_SIZE")
    write = _pmc_rows(write_csv, "WRITE_SIZE")

    def calib(rows):
        copies = [v for (name, v) in rows.values() if "copyBuffer" in name]
        return COPY_BYTES / (max(copies) * 1024.0)

    fs, ws = calib(fetch), calib(write)
    out = {}
    # (profile key, kernels whose traffic counts, kernels that mark one call, sources)
    for key, parts, primary, srcs in (
            ("attn_fwd_gqa_128k", ("attn_fwd_bf16_kernel",), ("attn_fwd_bf16_kernel",),
             ["attn_bf16.hip", "msa_plan.hpp", "msa_device.hpp"]),
            ("decode_512k", ("decode_fused_kernel", "decode_split_kernel", "decode_merge_kernel"),
             ("decode_fused_kernel", "decode_split_kernel"), ["decode.hip", "msa_plan.hpp", "msa_device.hpp"])):
        def total(rows):
            return sum(v for (name, v) in rows.values() if any(p in name for p in parts))

        def calls(rows):
            return max(1, sum(1 for (name, _) in rows.values() if any(p in name for p in primary)))

        fb = total(fetch) * 1024.0 * fs / calls(fetch)
        wb = total(write) * 1024.0 * ws / calls(write)
        rec = {"source_hash": kernel_hash(*srcs), "fetch_bytes": fb, "write_bytes": wb,
               "bytes_per_launch": fb + wb, "fetch_scale": fs, "write_scale": ws, "launches": calls(fetch)}
        with open(os.path.join(ROOT, "profiles", f"traffic_{key}.json"), "w") as f:
            json.dump(rec, f, indent=1)
        out[key] = rec
    # pooling: the cache's landmarks (137 GB read) and the prefill's (0.54 GB), told apart by size
    pf = {d: v for d, (name, v) in fetch.items() if "pool_kernel" in name}
    pw = {d: v for d, (name, v) in write.items() if "pool_kernel" in name}
    for key, big in (("pool_cache_512k", True), ("pool_prefill_128k", False)):
        fd = [v * 1024.0 * fs for v in pf.values() if (v * 1024.0 * fs > 1e10) == big]
        wd = [v * 1024.0 * ws for d, v in pw.items() if d in pf and (pf[d] * 1024.0 * fs > 1e10) == big]
        if not fd or not wd:
            continue
        rec = {"source_hash": kernel_hash("pool.hip", "msa_device.hpp"), "fetch_bytes": sum(fd) / len(fd),
               "write_bytes": sum(wd) / len(wd), "bytes_per_launch": sum(fd) / len(fd) + sum(wd) / len(wd),
               "fetch_scale": fs, "write_scale": ws, "launches": len(fd)}
        with open(os.path.join(ROOT, "profiles", f"traffic_{key}.json"), "w") as f:
            json.dump(rec, f, indent=1)
        out[key] = rec
    print(json.dumps(out, indent=1))


ATTN_SRCS = ["attn_bf16.hip", "msa_plan.hpp", "msa_device.hpp"]


def summarize_util(csv_path):
    """Matrix-core utilisation and shader clock of the 128K prefill kernel
    from a rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE run of
    this bench: busy cycles over (1024 SIMDs x cycles of the launch), at the
    clock the launch actually ran (GRBM_GUI_ACTIVE is summed over the 8
    XCDs) and at the 2.4 GHz nominal clock."""
    import csv

    per = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if "attn_fwd_bf16_kernel<128, true>" not in r["Kernel_Name"]:
                continue
            d = per.setdefault(r["Dispatch_Id"], {"ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
            d[r["Counter_Name"]] = float(r["Counter_Value"])
    rows = [d for d in per.values() if "SQ_VALU_MFMA_BUSY_CYCLES" in d and "GRBM_GUI_ACTIVE" in d]
    busy = sum(d["SQ_VALU_MFMA_BUSY_CYCLES"] for d in rows) / len(rows)
    cyc = sum(d["GRBM_GUI_ACTIVE"] / 8.0 for d in rows) / len(rows)
    ns = sum(d["ns"] for d in rows) / len(rows)
    rec = {"source_hash": kernel_hash(*ATTN_SRCS), "launches": len(rows), "launch_ms": ns / 1e6,
           "clock_ghz": cyc / ns, "mfma_busy_cycles": busy,
           "mfma_util_at_clock": busy / (1024.0 * cyc), "mfma_util_at_nominal": busy / (1024.0 * 2.4 * ns)}
    with open(os.path.join(ROOT, "profiles", "util_attn_fwd_gqa_128k.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def util_from_profiles():
    """The prefill's matrix-core utilisation from the committed counter
    summary, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "util_attn_fwd_gqa_128k.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_hash(*ATTN_SRCS):
        return None
    return {k: round(rec[k], 4) for k in ("mfma_util_at_clock", "mfma_util_at_nominal", "clock_ghz")}


def visible_pairs(n, w, G):
    import numpy as np
    import long_context_sparse_msa_amd as msa

    win_lo, lm = msa.msa_plan_rows(msa.attn_desc(1, 1, 1, n, 128, w, G))
    i = np.arange(n, dtype=np.int64)
    return int((i - win_lo + 1).sum()), int(lm.astype(np.int64).sum())


def cpu_baseline(cfg, Q, K, V, rows_per_head, heads):
    """Time the fp64 oracle on a bounded sample of the prefill workload."""
    import numpy as np
    import torch

    import msa_inputs as wl
    from oracle import msa_oracle as orc

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = len(os.sched_getaffinity(0))
    n, d, w, G = cfg.seq_len, cfg.head_dim, cfg.window, cfg.num_landmarks
    L = n // G
    g = heads[0] // (cfg.heads_q // cfg.heads_kv)
    Kh = K[:, g:g + 1].float().cpu().numpy().astype(np.float64)
    Vh = V[:, g:g + 1].float().cpu().numpy().astype(np.float64)
    rows = {h: np.sort(wl.sample_rows(n, h, rows_per_head, w, L)) for h in heads}
    Qr = {h: Q[:, h].index_select(1, torch.from_numpy(r).to(Q.device)).float().cpu().numpy().astype(np.float64)
          for h, r in rows.items()}
    pairs = 0
    for r in rows.values():
        pairs += int((np.minimum(r + 1, w)).sum())
        t = r - w + 1
        pairs += int(np.clip(np.where(t >= L, t // L, 0), 0, G).sum())
    t0 = time.perf_counter()
    Kb = orc.pool(Kh, G)
    Vb = orc.pool(Vh, G)
    for h, r in rows.items():
        Qfull = np.zeros((1, 1, n, d))
        Qfull[:, 0, r] = Qr[h]
        orc.attn(Qfull, Kh, Vh, w, G, cfg.scale, rows={0: r}, Kbar=Kb, Vbar=Vb)
    dt = time.perf_counter() - t0
    flops = 4.0 * d * pairs
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{cfg.name}: {len(heads)} query heads x {rows_per_head} seeded rows "
                  f"(+edge rows) of KV head {g}, fp64 numpy, landmark pooling included; "
                  f"{dt:.1f} s for {flops:.3e} useful FLOPs",
        "tiny_fp32_full": cpu_tiny_full(threads),
    }


def cpu_tiny_full(threads):
    """The whole fp64 oracle on the tiny fp32 workload (every row of every
    head), on all BLAS threads and on one."""
    import msa_inputs as wl
    from oracle import msa_oracle as orc

    cfg = wl.TINY_FP32
    q, k, v = (x.astype("float64") for x in wl.host_prefill_inputs(cfg))
    win, lm = visible_pairs(cfg.seq_len, cfg.window, cfg.num_landmarks)
    flops = 4.0 * cfg.head_dim * (win + lm) * cfg.heads_q * cfg.batch

    def run():
        t0 = time.perf_counter()
        orc.attn(q, k, v, cfg.window, cfg.num_landmarks, cfg.scale)
        return time.perf_counter() - t0

    t_all = min(run() for _ in range(2))
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(1):
            t_one = min(run() for _ in range(2))
    except ImportError:
        t_one = None
    return {
        "seconds": round(t_all, 4), "threads": int(threads),
        "TFLOP/s": flops / t_all / 1e12,
        "seconds_1_thread": None if t_one is None else round(t_one, 4),
        "TFLOP/s_1_thread": None if t_one is None else flops / t_one / 1e12,
        "flops": flops,
    }


def prefill_1m(torch, msa, wl, dev, stream, reps=3):
    """Secondary line: pooling + prefill of the 1M-token GQA workload."""
    cfg = wl.GQA_1M
    Q, K, V = wl.device_prefill_inputs(cfg, dev)
    G = cfg.num_landmarks
    Kb = torch.empty((cfg.batch, cfg.heads_kv, G, cfg.head_dim), dtype=torch.bfloat16, device=dev)
    Vb = torch.empty_like(Kb)
    O = torch.empty(Q.shape, dtype=torch.bfloat16, device=dev)
    LSE = torch.empty(Q.shape[:3], dtype=torch.float32, device=dev)
    run = lambda: (msa.msa_pool_landmarks(K, V, G, Kb, Vb),
                   msa.msa_attn_fwd(Q, K, V, Kb, Vb, cfg.window, G, cfg.scale, O=O, LSE=LSE))
    run()
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    e[0].record(stream)
    for _ in range(reps):
        run()
    e[1].record(stream)
    torch.cuda.synchronize()
    ms = e[0].elapsed_time(e[1]) / reps
    win, lm = visible_pairs(cfg.seq_len, cfg.window, G)
    flops = 4.0 * cfg.head_dim * (win + lm) * cfg.heads_q * cfg.batch
    del Q, K, V, O, LSE, Kb, Vb
    torch.cuda.empty_cache()
    return {"workload": "gqa_1m (n=1048576, 64/8 heads, d=128, w=4096, G=512), pooling + prefill",
            "ms": round(ms, 3), "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 2),
            "frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4), "launches": reps}


def incremental_decode(torch, msa, wl, dec, dev, stream, q, Kc, Vc, Kbc, Vbc, ws, Od, Ld, flush, flush_sink,
                       reps=5):
    """Secondary line: one serving step on the decode caches holding
    sequences of different lengths (seeded, uniform in [ctx/2, ctx]): append
    one token per sequence (msa_append_kv), then decode every sequence at
    its new length (msa_decode_fwd_varlen), the last-level cache flushed by
    a read before each decode.  The appended row is the same at every
    repetition, so the state does not drift.  Also times an append in which
    every sequence completes a landmark block (its worst case)."""
    lens = wl.decode_lengths(dec.batch, dec.ctx_len - 1)          # room for the appended token
    pos_d = torch.from_numpy(lens).to(dev)
    lens_d = pos_d + 1
    B, Hkv, d = dec.batch, dec.heads_kv, dec.head_dim
    k_new = torch.randn((B, Hkv, d), device=dev).to(torch.bfloat16)
    v_new = torch.randn((B, Hkv, d), device=dev).to(torch.bfloat16)
    G = dec.num_landmarks
    L = dec.ctx_len // G
    block_end = torch.from_numpy(((lens // L) * L + L - 1).astype("int32")).to(dev)  # completes a block

    def once(ev):
        torch.sum(flush, dim=(0,), dtype=torch.float32, out=flush_sink)
        ev[0].record(stream)
        msa.msa_append_kv(k_new, v_new, pos_d, Kc, Vc, Kbc, Vbc, G)
        ev[1].record(stream)
        msa.msa_decode_fwd_varlen(q, Kc, Vc, Kbc, Vbc, lens_d, dec.window, G, dec.num_splits, dec.scale,
                                  workspace=ws, O=Od, LSE=Ld)
        ev[2].record(stream)
        msa.msa_append_kv(k_new, v_new, block_end, Kc, Vc, Kbc, Vbc, G)
        ev[3].record(stream)

    once([torch.cuda.Event(enable_timing=True) for _ in range(4)])
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
    for ev in evs:
        once(ev)
    torch.cuda.synchronize()
    app = sum(e[0].elapsed_time(e[1]) for e in evs) / reps
    dms = sum(e[1].elapsed_time(e[2]) for e in evs) / reps
    blk = sum(e[2].elapsed_time(e[3]) for e in evs) / reps
    ddesc = msa.decode_desc(B, dec.heads_q, Hkv, dec.ctx_len, d, dec.window, G, dec.num_splits)
    entries = sum(msa.msa_plan_decode_varlen(ddesc, int(n) + 1)[2] for n in lens)
    nbytes = Hkv * entries * d * 2 * 2 + B * dec.heads_q * (d * 2 * 2 + 4)
    gbs = nbytes / (dms * 1e-3) / 1e9
    return {"workload": f"{B} sequences in a {dec.ctx_len}-token cache, lengths uniform in "
                        f"[{dec.ctx_len // 2}, {dec.ctx_len}) (seeded), {dec.num_splits} chunks; "
                        "append one token per sequence, then decode at the new lengths",
            "decode_ms": round(dms, 4), "decode_GBps": round(gbs, 1),
            "decode_frac": round(gbs / PEAK_HBM_GBS, 4), "bytes_per_launch": nbytes,
            "mean_length": round(float(lens.mean()) + 1, 1),
            "append_ms": round(app, 4), "append_block_ms": round(blk, 4),
            "append_block_bytes": int(B * Hkv * 2 * L * d * 2), "launches": reps}


def backward_128k(torch, msa, wl, dev, stream, reps=3):
    """Secondary line: the backward (msa_attn_bwd: dQ, dK, dV) of the 128K
    GQA prefill, from the forward's own O and LSE, dO ~ N(0, 1).  FLOPs are
    counted the usual way for attention backward, 2.5x the forward's: five
    products per visible pair (S recomputed, dP, dV, dK, dQ), 10*d FLOPs."""
    cfg = wl.GQA_128K
    Q, K, V = wl.device_prefill_inputs(cfg, dev)
    G = cfg.num_landmarks
    dO = torch.randn(Q.shape, device=dev).to(torch.bfloat16)
    Kb, Vb = msa.msa_pool_landmarks(K, V, G)
    O, LSE = msa.msa_attn_fwd(Q, K, V, Kb, Vb, cfg.window, G, cfg.scale)
    desc = msa.attn_desc(cfg.batch, cfg.heads_q, cfg.heads_kv, cfg.seq_len, cfg.head_dim, cfg.window, G,
                         cfg.scale, msa.MSA_DTYPE_BF16, msa.MSA_DTYPE_BF16)
    ws = torch.empty(msa.msa_attn_bwd_workspace_size(desc), dtype=torch.uint8, device=dev)
    dQ = torch.empty_like(Q)
    dK = torch.empty_like(K)
    dV = torch.empty_like(V)
    run = lambda: msa.msa_attn_bwd(Q, K, V, Kb, Vb, O, LSE, dO, cfg.window, G, cfg.scale,
                                   out_dtype=torch.bfloat16, workspace=ws, dQ=dQ, dK=dK, dV=dV)
    run()
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    e[0].record(stream)
    for _ in range(reps):
        run()
    e[1].record(stream)
    torch.cuda.synchronize()
    ms = e[0].elapsed_time(e[1]) / reps
    win, lm = visible_pairs(cfg.seq_len, cfg.window, G)
    flops = 10.0 * cfg.head_dim * (win + lm) * cfg.heads_q * cfg.batch
    del Q, K, V, dO, O, LSE, Kb, Vb, ws, dQ, dK, dV
    torch.cuda.empty_cache()
    return {"workload": "gqa_128k backward (n=131072, 64/8 heads, d=128, w=4096, G=512), dQ/dK/dV bf16",
            "ms": round(ms, 3), "flops_per_launch": flops, "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 2),
            "frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4), "launches": reps}


def blocksparse_band_128k(torch, msa, wl, dev, stream, reps=3):
    """Secondary line: msa_attn_fwd_blocksparse on the 128K GQA shapes with
    the band pattern of 128-token blocks each attending to the 16 blocks
    around it (non-causal).  FLOPs: 4*d per (row, listed key) pair."""
    cfg = wl.GQA_128K
    Q, K, V = wl.device_prefill_inputs(cfg, dev)
    counts, idx = wl.band_block_lists(cfg.batch, cfg.heads_q, cfg.seq_len)
    cd, id_ = torch.from_numpy(counts).to(dev), torch.from_numpy(idx).to(dev)
    O = torch.empty_like(Q)
    LSE = torch.empty(Q.shape[:3], dtype=torch.float32, device=dev)
    run = lambda: msa.msa_attn_fwd_blocksparse(Q, K, V, cd, id_, False, cfg.scale, O=O, LSE=LSE)
    run()
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    e[0].record(stream)
    for _ in range(reps):
        run()
    e[1].record(stream)
    torch.cuda.synchronize()
    ms = e[0].elapsed_time(e[1]) / reps
    n = cfg.seq_len
    keys_per_tile = [sum(min(n, (kb + 1) * 64) - kb * 64 for kb in idx[0, 0, t, :counts[0, 0, t]])
                     for t in range(counts.shape[2])]
    rows_per_tile = [min(n, (t + 1) * 128) - t * 128 for t in range(counts.shape[2])]
    pairs = sum(k * r for k, r in zip(keys_per_tile, rows_per_tile))
    flops = 4.0 * cfg.head_dim * pairs * cfg.heads_q * cfg.batch
    del Q, K, V, O, LSE, cd, id_
    torch.cuda.empty_cache()
    return {"workload": "gqa_128k shapes, block-sparse lists: each 128-token block attends to the 16 blocks "
                        "around it (non-causal)", "ms": round(ms, 3), "flops_per_launch": flops,
            "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 2),
            "frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4), "launches": reps}


def blocksparse_global_local_128k(torch, msa, wl, dev, stream, reps=3):
    """Secondary line: msa_attn_fwd_blocksparse on the 128K GQA shapes with
    global + local lists (non-causal): the first two 128-token blocks attend
    to every key and every block attends to them; the other blocks see a
    16-block local band.  FLOPs: 4*d per (row, listed key) pair."""
    cfg = wl.GQA_128K
    Q, K, V = wl.device_prefill_inputs(cfg, dev)
    counts, idx = wl.global_local_block_lists(cfg.batch, cfg.heads_q, cfg.seq_len)
    cd, id_ = torch.from_numpy(counts).to(dev), torch.from_numpy(idx).to(dev)
    O = torch.empty_like(Q)
    LSE = torch.empty(Q.shape[:3], dtype=torch.float32, device=dev)
    run = lambda: msa.msa_attn_fwd_blocksparse(Q, K, V, cd, id_, False, cfg.scale, O=O, LSE=LSE)
    run()
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    e[0].record(stream)
    for _ in range(reps):
        run()
    e[1].record(stream)
    torch.cuda.synchronize()
    ms = e[0].elapsed_time(e[1]) / reps
    n = cfg.seq_len
    rows_per_tile = [min(n, (t + 1) * 128) - t * 128 for t in range(counts.shape[2])]
    keys_per_tile = [sum(min(n, (kb + 1) * 64) - kb * 64 for kb in idx[0, 0, t, :counts[0, 0, t]])
                     for t in range(counts.shape[2])]
    pairs = sum(k * r for k, r in zip(keys_per_tile, rows_per_tile))
    flops = 4.0 * cfg.head_dim * pairs * cfg.heads_q * cfg.batch
    del Q, K, V, O, LSE, cd, id_
    torch.cuda.empty_cache()
    return {"workload": "gqa_128k shapes, block-sparse lists: global + local (2 global 128-token blocks that attend "
                        "to all and are attended by all, 16-block local band, non-causal)", "ms": round(ms, 3),
            "flops_per_launch": flops, "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 2),
            "frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4), "launches": reps}


def paged_decode(torch, msa, wl, dev, stream, page=64, reps=5):
    """Secondary line: the incremental-decode step on paged caches -- pools of
    64-row pages, each sequence's pages scattered by a seeded permutation --
    at the decode workload's shapes and the same seeded lengths: append one
    token per sequence, then decode (last-level cache flushed by a read
    before each decode)."""
    dec = wl.DECODE_512K
    B, Hq, Hkv, C, d, G = dec.batch, dec.heads_q, dec.heads_kv, dec.ctx_len, dec.head_dim, dec.num_landmarks
    P = C // page
    n_pages = B * P
    Kp = torch.empty((n_pages, Hkv, page, d), dtype=torch.bfloat16, device=dev).normal_()
    Vp = torch.empty_like(Kp).normal_()
    perm = torch.from_numpy(__import__("numpy").random.default_rng(7).permutation(n_pages).reshape(B, P)
                            .astype("int32")).to(dev)
    Kb = torch.randn((B, Hkv, G, d), device=dev).to(torch.bfloat16)
    Vb = torch.randn((B, Hkv, G, d), device=dev).to(torch.bfloat16)
    q = torch.randn((B, Hq, d), device=dev).to(torch.bfloat16)
    lens = wl.decode_lengths(B, C - 1)
    pos_d = torch.from_numpy(lens).to(dev)
    lens_d = pos_d + 1
    k_new = torch.randn((B, Hkv, d), device=dev).to(torch.bfloat16)
    v_new = torch.randn((B, Hkv, d), device=dev).to(torch.bfloat16)
    ddesc = msa.decode_desc(B, Hq, Hkv, C, d, dec.window, G, dec.num_splits)
    ws = torch.empty(msa.msa_decode_workspace_size(ddesc) // 4, dtype=torch.float32, device=dev)
    O = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=dev)
    LSE = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    flush = torch.empty(1 << 28, dtype=torch.float16, device=dev).fill_(1.0)
    sink = torch.empty((), dtype=torch.float32, device=dev)

    def once(ev):
        torch.sum(flush, dim=(0,), dtype=torch.float32, out=sink)
        ev[0].record(stream)
        msa.msa_append_kv_paged(k_new, v_new, pos_d, Kp, Vp, perm, Kb, Vb, G)
        ev[1].record(stream)
        msa.msa_decode_fwd_paged(q, Kp, Vp, perm, Kb, Vb, lens_d, dec.window, G, dec.num_splits, dec.scale,
                                 workspace=ws, O=O, LSE=LSE)
        ev[2].record(stream)

    once([torch.cuda.Event(enable_timing=True) for _ in range(3)])
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    for ev in evs:
        once(ev)
    torch.cuda.synchronize()
    app = sum(e[0].elapsed_time(e[1]) for e in evs) / reps
    dms = sum(e[1].elapsed_time(e[2]) for e in evs) / reps
    entries = sum(msa.msa_plan_decode_varlen(ddesc, int(n) + 1)[2] for n in lens)
    nbytes = Hkv * entries * d * 2 * 2 + B * Hq * (d * 2 * 2 + 4)
    gbs = nbytes / (dms * 1e-3) / 1e9
    del Kp, Vp, perm, Kb, Vb, q, ws, O, LSE, flush, sink
    torch.cuda.empty_cache()
    return {"workload": f"paged caches ({page}-row pages, pages of each sequence scattered by a seeded "
                        f"permutation), {B} sequences, capacity {C}, same lengths as incremental_decode",
            "decode_ms": round(dms, 4), "decode_GBps": round(gbs, 1), "decode_frac": round(gbs / PEAK_HBM_GBS, 4),
            "bytes_per_launch": nbytes, "append_ms": round(app, 4), "launches": reps}


def mfma_references():
    """Matrix-core throughput of two fixed instruction streams, run by
    libmsa_ref.so on this GPU (2048 workgroups, two wavefronts per SIMD,
    random bf16 operands, best of 5 launches): MFMAs on register operands,
    and the prefill's per-tile chain QK -> softmax -> PV with its LDS operand
    reads and no HBM traffic."""
    import ctypes

    path = os.path.join(ROOT, "long_context_sparse_msa_amd", "libmsa_ref.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: run long_context_sparse_msa_amd.build first")
    lib = ctypes.CDLL(path)
    lib.msa_ref_mfma.restype = ctypes.c_int
    lib.msa_ref_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                 ctypes.POINTER(ctypes.c_double)]
    out = {}
    for mode, key in ((0, "mfma_register_tflops"), (1, "mfma_chain_tflops")):
        ms, flops = ctypes.c_double(), ctypes.c_double()
        rc = lib.msa_ref_mfma(mode, 2000, 5, ctypes.byref(ms), ctypes.byref(flops))
        if rc != 0:
            raise RuntimeError(f"msa_ref_mfma(mode {mode}) failed with HIP error {rc}")
        out[key] = round(flops.value / (ms.value * 1e-3) / 1e12, 1)
    out["mfma_register"] = "32x32x16 bf16 MFMAs on register operands, four accumulators"
    out["mfma_chain"] = ("per trip QK (16 MFMAs, A by ds_read_b128) -> exp2 of the 32 scores per lane, sums, "
                         "packs, dot products -> PV (16 MFMAs, A by transpose reads), no HBM traffic")
    return out


def measured_peaks(torch, dev, reps=10):
    """Achievable references on this GPU through vendor libraries: a large
    bf16 GEMM (hipBLASLt) and a 2 GiB device copy (bytes read + written)."""
    a = torch.randn((8192, 8192), dtype=torch.bfloat16, device=dev)
    b = torch.randn((8192, 8192), dtype=torch.bfloat16, device=dev)
    c = torch.empty((8192, 8192), dtype=torch.bfloat16, device=dev)
    torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    e[0].record()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    e[1].record()
    torch.cuda.synchronize()
    gemm = 2.0 * 8192 ** 3 / (e[0].elapsed_time(e[1]) / reps * 1e-3) / 1e12
    del a, b, c
    x = torch.empty(1 << 30, dtype=torch.bfloat16, device=dev).fill_(1.0)
    y = torch.empty_like(x)
    y.copy_(x)
    torch.cuda.synchronize()
    e[0].record()
    for _ in range(reps):
        y.copy_(x)
    e[1].record()
    torch.cuda.synchronize()
    copy = 2.0 * x.numel() * 2 / (e[0].elapsed_time(e[1]) / reps * 1e-3) / 1e9
    del y
    # read-only stream: float32-accumulated sums of the same 2 GiB taken as rows
    # of 4096 (one float written per 8 KB read; the fastest of the torch
    # reductions tried, against 3.6 TB/s for one sum over the whole buffer)
    xv = x.view(-1, 4096)
    sink = torch.empty(xv.shape[0], dtype=torch.float32, device=dev)
    torch.sum(xv, dim=1, dtype=torch.float32, out=sink)
    torch.cuda.synchronize()
    e[0].record()
    for _ in range(reps):
        torch.sum(xv, dim=1, dtype=torch.float32, out=sink)
    e[1].record()
    torch.cuda.synchronize()
    read = x.numel() * 2 / (e[0].elapsed_time(e[1]) / reps * 1e-3) / 1e9
    del x, xv, sink
    torch.cuda.empty_cache()
    torch.cuda.synchronize()
    refs = mfma_references()
    return {**refs, "bf16_gemm_tflops": round(gemm, 1), "bf16_gemm_shape": "8192^3 (torch.matmul)",
            "hbm_copy_gbs": round(copy, 1), "hbm_copy": "2 GiB device copy, read + write bytes",
            "hbm_read_gbs": round(read, 1), "hbm_read": "float32-accumulated torch.sum over 2 GiB of bf16 in rows of 4096, bytes read"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=49152, help="oracle rows per head for the CPU baseline")
    ap.add_argument("--no-1m", action="store_true", help="skip the secondary 1M-token prefill measurement")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured achievable-peak reference runs")
    ap.add_argument("--no-backward", action="store_true", help="skip the secondary backward measurement")
    ap.add_argument("--no-blocksparse", action="store_true",
                    help="skip the secondary block-sparse-list measurement")
    ap.add_argument("--no-incremental", action="store_true",
                    help="skip the secondary incremental-decode (append + varlen decode) measurement")
    ap.add_argument("--paged-only", action="store_true",
                    help="run only the paged-decode line, in a process that has allocated nothing else "
                         "(the default run allocates and frees the 137 GB contiguous caches first)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a 1 GiB device-to-device copy before timing (reference dispatch for HBM counters)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn rocprofv3 FETCH_SIZE / WRITE_SIZE counter CSVs of a bench run into "
                         "profiles/traffic_*.json and print the summary; runs nothing on the GPU")
    ap.add_argument("--summarize-util", metavar="CSV",
                    help="turn a rocprofv3 SQ_VALU_MFMA_BUSY_CYCLES / GRBM_GUI_ACTIVE counter CSV of a bench run "
                         "into profiles/util_attn_fwd_gqa_128k.json; runs nothing on the GPU")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_util:
        summarize_util(args.summarize_util)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import long_context_sparse_msa_amd as msa
    import msa_inputs as wl

    dev = torch.device("cuda:0")
    pre, dec = wl.GQA_128K, wl.DECODE_512K
    stream = torch.cuda.current_stream(dev)
    if args.paged_only:
        print(json.dumps({"paged_decode_fresh_process": paged_decode(torch, msa, wl, dev, stream)}), flush=True)
        return
    if args.calibrate_copy:
        x = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
        y = torch.empty_like(x)
        y.copy_(x)
        torch.cuda.synchronize()
        del x, y

    # ---- inputs, resident in HBM before anything is timed
    Q, K, V = wl.device_prefill_inputs(pre, dev)
    B, Hq, Hkv, n, d = pre.batch, pre.heads_q, pre.heads_kv, pre.seq_len, pre.head_dim
    G = pre.num_landmarks
    Kb = torch.empty((B, Hkv, G, d), dtype=torch.bfloat16, device=dev)
    Vb = torch.empty_like(Kb)
    O = torch.empty((B, Hq, n, d), dtype=torch.bfloat16, device=dev)
    LSE = torch.empty((B, Hq, n), dtype=torch.float32, device=dev)

    q, Kc, Vc = wl.device_decode_inputs(dec, dev)
    Kbc = torch.empty((dec.batch, dec.heads_kv, dec.num_landmarks, d), dtype=torch.bfloat16, device=dev)
    Vbc = torch.empty_like(Kbc)
    ddesc = msa.decode_desc(dec.batch, dec.heads_q, dec.heads_kv, dec.ctx_len, d, dec.window,
                            dec.num_landmarks, dec.num_splits)
    ws = torch.empty(msa.msa_decode_workspace_size(ddesc) // 4, dtype=torch.float32, device=dev)
    Od = torch.empty((dec.batch, dec.heads_q, d), dtype=torch.bfloat16, device=dev)
    Ld = torch.empty((dec.batch, dec.heads_q), dtype=torch.float32, device=dev)

    # cache landmarks (static across decode steps): pooled once, timed once
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    msa.msa_pool_landmarks(Kc, Vc, dec.num_landmarks, Kbc, Vbc)
    e0.record(stream)
    msa.msa_pool_landmarks(Kc, Vc, dec.num_landmarks, Kbc, Vbc)
    e1.record(stream)
    torch.cuda.synchronize()
    cache_pool_ms = e0.elapsed_time(e1)
    cache_bytes = 2 * Kc.numel() * 2 + 2 * Kbc.numel() * 2

    # 512 MiB read (not written: evicting dirty lines would slow the decode
    # that follows) before each decode call, so the 256 MB last-level cache
    # holds nothing of the cache the decode streams
    flush = torch.empty(1 << 28, dtype=torch.float16, device=dev).fill_(1.0)
    flush_sink = torch.empty((), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step(ev):
        ev[0].record(stream)
        msa.msa_pool_landmarks(K, V, G, Kb, Vb)
        ev[1].record(stream)
        msa.msa_attn_fwd(Q, K, V, Kb, Vb, pre.window, G, pre.scale, O=O, LSE=LSE)
        ev[2].record(stream)
        torch.sum(flush, dim=(0,), dtype=torch.float32, out=flush_sink)
        ev[3].record(stream)
        msa.msa_decode_fwd(q, Kc, Vc, Kbc, Vbc, dec.window, dec.num_landmarks, dec.num_splits, dec.scale,
                           workspace=ws, O=Od, LSE=Ld)
        ev[4].record(stream)

    for _ in range(args.warmup):
        step([torch.cuda.Event(enable_timing=True) for _ in range(5)])
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    # pooling alone, launched back to back: for a 0.1 ms kernel the event pair
    # around one launch inside the step adds several microseconds
    b2b = 20
    e0.record(stream)
    for _ in range(b2b):
        msa.msa_pool_landmarks(K, V, G, Kb, Vb)
    e1.record(stream)
    torch.cuda.synchronize()
    pool_b2b_ms = e0.elapsed_time(e1) / b2b
    pool_t = [e[0].elapsed_time(e[1]) for e in evs]
    attn_t = [e[1].elapsed_time(e[2]) for e in evs]
    dec_t = [e[3].elapsed_time(e[4]) for e in evs]
    pool_ms = sum(pool_t) / args.steps
    attn_ms = sum(attn_t) / args.steps
    dec_ms = sum(dec_t) / args.steps

    def stats(ts):
        ts = sorted(ts)
        return {"mean": round(sum(ts) / len(ts), 4), "median": round(ts[len(ts) // 2], 4), "min": round(ts[0], 4)}

    # ---- algorithmic work
    win_pairs, lm_pairs = visible_pairs(n, pre.window, G)
    flops = 4.0 * d * (win_pairs + lm_pairs) * Hq * B
    pool_bytes = 2 * K.numel() * 2 + 2 * Kb.numel() * 2
    dp = msa.msa_plan_decode(ddesc)
    entries = dp[2]
    dec_bytes = (dec.batch * dec.heads_kv * entries * d * 2 * 2      # K and V rows (window + landmarks)
                 + dec.batch * dec.heads_q * d * 2 * 2               # q in, O out
                 + dec.batch * dec.heads_q * 4)                      # LSE out

    prefill_tflops = flops / ((pool_ms + attn_ms) * 1e-3) / 1e12
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    dec_gbs = dec_bytes / (dec_ms * 1e-3) / 1e9

    out = {
        "metric": METRIC,
        "value": round(prefill_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "gqa_128k prefill (landmark pooling + sparse attention) + decode_512k "
                        "(split-KV, 16 chunks, LSE merge)",
            "batch": B, "seq_len": n, "heads_q": Hq, "heads_kv": Hkv, "head_dim": d,
            "window": pre.window, "landmarks": G,
            "decode_batch": dec.batch, "decode_ctx": dec.ctx_len, "decode_splits": dec.num_splits,
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_fwd_bf16_kernel<128, bf16 out>",
            "achieved": round(attn_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic_from_profiles("attn_fwd_gqa_128k", ATTN_SRCS),
            "mfma_util": util_from_profiles(),
            "flops_per_launch": flops,
            "avg_launch_ms": round(attn_ms, 4),
        },
        "decode": {
            "value": round(dec_gbs, 1),
            "unit": "GB/s",
            "ms": round(dec_ms, 4),
            "roofline": {
                "bound": "hbm", "achieved": round(dec_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(dec_gbs / PEAK_HBM_GBS, 4), "bytes_per_launch": dec_bytes,
                "traffic": traffic_from_profiles("decode_512k", ["decode.hip", "msa_plan.hpp",
                                                                 "msa_device.hpp"]),
            },
        },
        "pool": {
            "prefill_ms": round(pool_ms, 4),
            "prefill_GBps": round(pool_bytes / (pool_ms * 1e-3) / 1e9, 1),
            "prefill_bytes_per_launch": pool_bytes,
            "prefill_ms_back_to_back": round(pool_b2b_ms, 4),
            "prefill_GBps_back_to_back": round(pool_bytes / (pool_b2b_ms * 1e-3) / 1e9, 1),
            "prefill_traffic": traffic_from_profiles("pool_prefill_128k", ["pool.hip", "msa_device.hpp"]),
            "cache_ms": round(cache_pool_ms, 4),
            "cache_GBps": round(cache_bytes / (cache_pool_ms * 1e-3) / 1e9, 1),
            "cache_bytes_per_launch": cache_bytes,
            "cache_traffic": traffic_from_profiles("pool_cache_512k", ["pool.hip", "msa_device.hpp"]),
        },
        "kernels_ms": {"pool": stats(pool_t), "attn_fwd": stats(attn_t), "decode": stats(dec_t)},
        "useful_pairs_per_head": {"window": win_pairs, "landmark": lm_pairs},
        "cpu_baseline": None,
    }

    if not args.no_incremental:
        out["incremental_decode"] = incremental_decode(torch, msa, wl, dec, dev, stream, q, Kc, Vc, Kbc, Vbc, ws,
                                                       Od, Ld, flush, flush_sink)
    del q, Kc, Vc, ws, flush, flush_sink
    torch.cuda.empty_cache()
    if not args.no_incremental:
        out["paged_decode"] = paged_decode(torch, msa, wl, dev, stream)
    if not args.no_1m:
        out["prefill_1m"] = prefill_1m(torch, msa, wl, dev, stream)
    if not args.no_backward:
        out["backward"] = backward_128k(torch, msa, wl, dev, stream)
    if not args.no_blocksparse:
        out["blocksparse"] = blocksparse_band_128k(torch, msa, wl, dev, stream)
        out["blocksparse_global_local"] = blocksparse_global_local_128k(torch, msa, wl, dev, stream)
    if not args.no_peaks:
        peaks = measured_peaks(torch, dev)
        out["measured_peaks"] = peaks
        out["roofline"]["frac_of_measured"] = round(attn_tflops / peaks["bf16_gemm_tflops"], 4)
        out["roofline"]["frac_of_chain"] = round(attn_tflops / peaks["mfma_chain_tflops"], 4)
        # decode only reads: its reference is the read-only stream
        out["decode"]["roofline"]["frac_of_measured"] = round(dec_gbs / peaks["hbm_read_gbs"], 4)
        out["decode"]["roofline"]["measured_reference"] = "hbm_read_gbs"
        out["pool"]["frac_of_measured_back_to_back"] = round(out["pool"]["prefill_GBps_back_to_back"] /
                                                             peaks["hbm_read_gbs"], 4)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(pre, Q, K, V, args.cpu_rows, list(range(8)))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
