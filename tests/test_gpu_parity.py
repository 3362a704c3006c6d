"""GPU parity: libmsa's kernels, called through the C ABI, against the fp64
oracle on the same seeded inputs.

Small problems are compared on every row; the workload shapes on 4096
seeded rows per head plus forced edge rows.  The float32 epilogue is
graded (see gpu_util for the bounds); the bf16 store must equal its
round-to-nearest-even exactly.
"""
import math
import os

import numpy as np
import pytest
import torch

import msa_inputs as wl
from oracle import msa_oracle as orc
from tests.gpu_util import TOL_BF16, TOL_F32, assert_close, bf16_rne, check_rows, dev, host64

pytestmark = pytest.mark.gpu

msa = pytest.importorskip("long_context_sparse_msa_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    msa.lib()  # a missing library is an error, not a skip
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def rand(shape, seed, dtype):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32).to(dtype).to(dev())


# ------------------------------------------------------------------ pooling

def ulp_bf16(x):
    x = np.abs(x)
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -126)))
    return 2.0 ** (e - 7)


@pytest.mark.parametrize("B,H,n,d,G,dt", [
    (1, 2, 2048, 64, 16, torch.float32), (2, 3, 640, 128, 5, torch.float32),
    (1, 8, 32768, 128, 512, torch.bfloat16), (2, 2, 1000, 128, 8, torch.bfloat16),
    (1, 4, 4096, 64, 4096, torch.bfloat16), (1, 1, 7, 128, 1, torch.bfloat16),
])
def test_pool(B, H, n, d, G, dt):
    print(f"[case] pool B={B} H={H} n={n} d={d} G={G} {dt}", flush=True)
    K = rand((B, H, n, d), 1, dt)
    V = rand((B, H, n, d), 2, dt)
    Kb, Vb = msa.msa_pool_landmarks(K, V, G)
    torch.cuda.synchronize()
    for src, out in ((K, Kb), (V, Vb)):
        ref = orc.pool(host64(src), G)
        got = host64(out)
        if dt == torch.float32:
            assert np.abs(got - ref).max() <= 1e-6
        else:
            assert (np.abs(got - ref) <= ulp_bf16(ref)).all()


def test_pool_workload_128k():
    cfg = wl.GQA_128K
    print("[case] pool gqa_128k", flush=True)
    _, K, V = wl.device_prefill_inputs(cfg, dev())
    Kb, Vb = msa.msa_pool_landmarks(K, V, cfg.num_landmarks)
    torch.cuda.synchronize()
    for src, out in ((K, Kb), (V, Vb)):
        ref = orc.pool(host64(src), cfg.num_landmarks)
        assert (np.abs(host64(out) - ref) <= ulp_bf16(ref)).all()


# ------------------------------------------------------------------ prefill, small, every row

def run_attn(Q, K, V, w, G, scale=None, out_dtype=None):
    Kb, Vb = msa.msa_pool_landmarks(K, V, G) if G else (None, None)
    O, LSE = msa.msa_attn_fwd(Q, K, V, Kb, Vb, w, G, scale, out_dtype=out_dtype)
    return O, LSE


def test_tiny_fp32_workload():
    cfg = wl.TINY_FP32
    print("[case] tiny_fp32", flush=True)
    q, k, v = wl.host_prefill_inputs(cfg)
    Q, K, V = (torch.from_numpy(x).to(dev()) for x in (q, k, v))
    O, LSE = run_attn(Q, K, V, cfg.window, cfg.num_landmarks, cfg.scale)
    torch.cuda.synchronize()
    o_ref, l_ref = orc.attn_dense(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                                  cfg.window, cfg.num_landmarks, cfg.scale)
    assert_close(host64(O), host64(LSE), o_ref, l_ref, TOL_F32, "tiny_fp32 all rows")


SMALL = [
    # B, Hq, Hkv, n, d, w, G
    (1, 2, 2, 256, 128, 64, 4),
    (2, 4, 2, 320, 128, 100, 5),      # ragged last query tile, GQA, batch 2
    (1, 2, 1, 200, 64, 50, 8),        # d = 64, n not a multiple of 64
    (1, 2, 2, 64, 128, 1, 0),         # w = 1, no landmarks: O = V
    (1, 2, 2, 384, 128, 1000, 0),     # window beyond n: causal attention
    (1, 2, 2, 256, 128, 7, 256),      # one-token landmarks: causal attention
    (1, 8, 1, 1100, 128, 300, 11),    # 8 query heads per KV head, L = 100
    (1, 1, 1, 1, 128, 1, 1),          # a single token
    (1, 2, 2, 4096, 128, 512, 64),
    (1, 16, 16, 130, 64, 130, 13),
]


@pytest.mark.parametrize("B,Hq,Hkv,n,d,w,G", SMALL)
def test_attn_small_bf16(B, Hq, Hkv, n, d, w, G):
    print(f"[case] attn bf16 B={B} Hq={Hq} Hkv={Hkv} n={n} d={d} w={w} G={G}", flush=True)
    Q = rand((B, Hq, n, d), 3, torch.bfloat16)
    K = rand((B, Hkv, n, d), 4, torch.bfloat16)
    V = rand((B, Hkv, n, d), 5, torch.bfloat16)
    scale = 1.0 / math.sqrt(d)
    O32, L32 = run_attn(Q, K, V, w, G, scale, out_dtype=torch.float32)
    O16, L16 = run_attn(Q, K, V, w, G, scale)
    torch.cuda.synchronize()
    o_ref, l_ref = orc.attn_dense(host64(Q), host64(K), host64(V), w, G, scale)
    assert_close(host64(O32), host64(L32), o_ref, l_ref, TOL_BF16, f"bf16 n={n} w={w} G={G}")
    assert torch.equal(O16, bf16_rne(O32)), "bf16 store is not RNE of the float32 epilogue"
    assert torch.equal(L16, L32)
    if w == 1 and G == 0:
        assert torch.equal(O32, V.float().repeat_interleave(Hq // Hkv, dim=1))


@pytest.mark.parametrize("spike", [0.0, 3.0], ids=["rising", "rising+spikes"])
def test_attn_rising_scores_bf16(spike):
    """Scores that keep climbing along every row's walk (coordinate 0 of K
    grows with the position and coordinate 0 of Q is 2), so the running
    reference max falls behind by more than 2^8 about three times per row
    after the first tile; with spikes (every 211th key row x3) a single
    score also overflows exp2 against the old reference on about one tile
    in ten rows.  The kernel's rescale-and-redo path runs often and must
    still match the oracle."""
    print(f"[case] attn bf16 rising scores spike={spike}", flush=True)
    B, Hq, Hkv, n, d, w, G = 1, 4, 2, 2048, 128, 640, 16
    Q = rand((B, Hq, n, d), 11, torch.float32)
    Q[..., 0] = 2.0
    Q = Q.to(torch.bfloat16)
    K = rand((B, Hkv, n, d), 12, torch.float32)
    K[..., 0] += 0.2 * torch.arange(n, dtype=torch.float32, device=K.device)
    if spike:
        K[:, :, torch.arange(37, n, 211, device=K.device)] *= spike
    K = K.to(torch.bfloat16)
    V = rand((B, Hkv, n, d), 13, torch.bfloat16)
    scale = 1.0 / math.sqrt(d)
    O32, L32 = run_attn(Q, K, V, w, G, scale, out_dtype=torch.float32)
    O16, L16 = run_attn(Q, K, V, w, G, scale)
    torch.cuda.synchronize()
    o_ref, l_ref = orc.attn_dense(host64(Q), host64(K), host64(V), w, G, scale)
    assert np.ptp(l_ref) > 40.0, "the case should span a wide range of row maxima"
    assert_close(host64(O32), host64(L32), o_ref, l_ref, TOL_BF16, f"bf16 rising scores spike={spike}")
    assert torch.equal(O16, bf16_rne(O32)), "bf16 store is not RNE of the float32 epilogue"
    assert torch.equal(L16, L32)


def test_attn_small_fp32_d128():
    print("[case] attn fp32 d=128", flush=True)
    B, Hq, Hkv, n, d, w, G = 1, 4, 2, 333, 128, 70, 9
    Q, K, V = (rand((B, h, n, d), s, torch.float32) for h, s in ((Hq, 6), (Hkv, 7), (Hkv, 8)))
    O, LSE = run_attn(Q, K, V, w, G, 0.1)
    torch.cuda.synchronize()
    o_ref, l_ref = orc.attn_dense(host64(Q), host64(K), host64(V), w, G, 0.1)
    assert_close(host64(O), host64(LSE), o_ref, l_ref, TOL_F32, "fp32 d=128")


# ------------------------------------------------------------------ prefill, workload shapes

def sampled(cfg):
    L = cfg.seq_len // cfg.num_landmarks
    return {h: wl.sample_rows(cfg.seq_len, h, 4096, cfg.window, L) for h in range(cfg.heads_q)}


def raw_bf16_report(O16, O32, cfg, rows_by_head):
    """Informational: the bf16 store's own distance to the float32 result."""
    d = (O16.float() - O32).abs()
    print(f"[info] {cfg.name}: bf16 store vs fp32 epilogue max {d.max().item():.3e} "
          f"mean {d.mean().item():.3e}", flush=True)


@pytest.mark.parametrize("cfg", [wl.BF16_32K, wl.BF16_32K_PEAKY], ids=lambda c: c.name)
def test_attn_32k(cfg):
    print(f"[case] {cfg.name}", flush=True)
    Q, K, V = wl.device_prefill_inputs(cfg, dev())
    O32, L32 = run_attn(Q, K, V, cfg.window, cfg.num_landmarks, cfg.scale, out_dtype=torch.float32)
    O16, L16 = run_attn(Q, K, V, cfg.window, cfg.num_landmarks, cfg.scale)
    O16b, L16b = run_attn(Q, K, V, cfg.window, cfg.num_landmarks, cfg.scale)
    torch.cuda.synchronize()
    assert torch.equal(O16, bf16_rne(O32))
    assert torch.equal(O16, O16b) and torch.equal(L16, L16b), "not deterministic"
    raw_bf16_report(O16, O32, cfg, None)
    check_rows(Q, K, V, O32, L32, cfg.window, cfg.num_landmarks, cfg.scale, sampled(cfg), TOL_BF16, cfg.name,
               O16=O16)


@pytest.fixture(scope="module")
def gqa128k():
    cfg = wl.GQA_128K
    print(f"[case] {cfg.name} (shared run)", flush=True)
    Q, K, V = wl.device_prefill_inputs(cfg, dev())
    O32, L32 = run_attn(Q, K, V, cfg.window, cfg.num_landmarks, cfg.scale, out_dtype=torch.float32)
    O16, _ = run_attn(Q, K, V, cfg.window, cfg.num_landmarks, cfg.scale)
    torch.cuda.synchronize()
    assert torch.equal(O16, bf16_rne(O32))
    yield cfg, Q, K, V, O32, L32, O16
    del Q, K, V, O32, L32, O16
    torch.cuda.empty_cache()


@pytest.mark.parametrize("g", range(8))
def test_attn_128k_kv_group(gqa128k, g):
    cfg, Q, K, V, O32, L32, O16 = gqa128k
    rows = {h: r for h, r in sampled(cfg).items() if h // 8 == g}
    check_rows(Q, K, V, O32, L32, cfg.window, cfg.num_landmarks, cfg.scale, rows, TOL_BF16,
               f"{cfg.name} kv{g}", O16=O16)


@pytest.fixture(scope="module")
def gqa1m():
    cfg = wl.GQA_1M
    print(f"[case] {cfg.name} (shared run)", flush=True)
    Q, K, V = wl.device_prefill_inputs(cfg, dev())
    O32, L32 = run_attn(Q, K, V, cfg.window, cfg.num_landmarks, cfg.scale, out_dtype=torch.float32)
    O16, _ = run_attn(Q, K, V, cfg.window, cfg.num_landmarks, cfg.scale)
    torch.cuda.synchronize()
    assert torch.equal(O16, bf16_rne(O32))
    yield cfg, Q, K, V, O32, L32, O16
    del Q, K, V, O32, L32, O16
    torch.cuda.empty_cache()


@pytest.mark.parametrize("g", range(8))
def test_attn_1m_kv_group(gqa1m, g):
    cfg, Q, K, V, O32, L32, O16 = gqa1m
    rows = {h: r for h, r in sampled(cfg).items() if h // 8 == g}
    check_rows(Q, K, V, O32, L32, cfg.window, cfg.num_landmarks, cfg.scale, rows, TOL_BF16,
               f"{cfg.name} kv{g}", group_span=4096, O16=O16)


def test_attn_compression_tokens_128k():
    """Landmarks at the pages' finer granularity: 256 compression tokens per
    8K chunk (L = 32, so G = n/32 = 4096 landmarks) at 128K tokens, one KV
    group of 8 query heads; rows sampled per head."""
    B, Hq, Hkv, n, d, w, G = 1, 8, 1, 131072, 128, 4096, 4096
    print(f"[case] compression tokens n={n} w={w} G={G}", flush=True)
    Q = rand((B, Hq, n, d), 21, torch.bfloat16)
    K = rand((B, Hkv, n, d), 22, torch.bfloat16)
    V = rand((B, Hkv, n, d), 23, torch.bfloat16)
    scale = 1.0 / math.sqrt(d)
    O32, L32 = run_attn(Q, K, V, w, G, scale, out_dtype=torch.float32)
    O16, _ = run_attn(Q, K, V, w, G, scale)
    torch.cuda.synchronize()
    assert torch.equal(O16, bf16_rne(O32))
    rows = {h: wl.sample_rows(n, h, 1024, w, n // G) for h in range(Hq)}
    check_rows(Q, K, V, O32, L32, w, G, scale, rows, TOL_BF16, "compression tokens 128k", group_span=4096)


# ------------------------------------------------------------------ decode

DEC = [
    # B, Hq, Hkv, ctx, d, w, G, S
    (2, 8, 2, 512, 128, 64, 8, 4),
    (1, 4, 4, 300, 128, 1000, 0, 3),    # window covers the whole cache, no landmarks
    (3, 16, 1, 1024, 64, 100, 16, 40),  # more chunks than entries allow: empty chunks
    (1, 8, 1, 64, 128, 8, 8, 16),
    (2, 2, 2, 1, 128, 1, 1, 2),         # a single cached token
    (1, 8, 8, 4096, 128, 300, 16, 7),
    (2, 6, 2, 2048, 128, 129, 32, 1),   # unsplit
    (2, 8, 1, 65536, 128, 4096, 2048, 16),  # 32-token landmarks (256 per 8K): 1920 visible
]


@pytest.mark.parametrize("schedule", ["split", "fused"])
@pytest.mark.parametrize("B,Hq,Hkv,ctx,d,w,G,S", DEC)
def test_decode_small(B, Hq, Hkv, ctx, d, w, G, S, schedule):
    print(f"[case] decode {schedule} B={B} Hq={Hq} Hkv={Hkv} ctx={ctx} d={d} w={w} G={G} S={S}", flush=True)
    q = rand((B, Hq, d), 9, torch.bfloat16)
    Kc = rand((B, Hkv, ctx, d), 10, torch.bfloat16)
    Vc = rand((B, Hkv, ctx, d), 11, torch.bfloat16)
    scale = 1.0 / math.sqrt(d)
    Kb, Vb = msa.msa_pool_landmarks(Kc, Vc, G) if G else (None, None)
    desc = msa.decode_desc(B, Hq, Hkv, ctx, d, w, G, S, scale, msa.MSA_DTYPE_BF16, msa.MSA_DTYPE_F32)
    ws = torch.empty(msa.msa_decode_workspace_size(desc) // 4, dtype=torch.float32, device=dev())
    O32, L32 = msa.msa_decode_fwd(q, Kc, Vc, Kb, Vb, w, G, S, scale, out_dtype=torch.float32, workspace=ws, schedule=schedule)
    po, pl = msa.decode_partials(ws, S, B, Hq, d)
    po, pl = host64(po), host64(pl)
    O16, L16 = msa.msa_decode_fwd(q, Kc, Vc, Kb, Vb, w, G, S, scale, schedule=schedule)
    torch.cuda.synchronize()
    q64, k64, v64 = host64(q), host64(Kc), host64(Vc)
    o_ref, l_ref = orc.decode(q64, k64, v64, w, G, scale)
    assert_close(host64(O32), host64(L32), o_ref, l_ref, TOL_BF16, "decode merged")
    assert torch.equal(O16, bf16_rne(O32))
    if schedule != "split":
        return  # the fused schedule keeps the partials on chip
    # Per-chunk partials.  A chunk may hold a single landmark, whose score the
    # bf16 storage of the pooled landmark moves by up to ~1e-3 at short
    # blocks; chunks are therefore graded against the oracle fed with its
    # own fp64 landmark means rounded to bf16 (the merged result above is
    # graded against the exact means).
    if G:
        kb_r = host64(torch.from_numpy(orc.pool(k64, G)).to(torch.bfloat16))
        vb_r = host64(torch.from_numpy(orc.pool(v64, G)).to(torch.bfloat16))
    else:
        kb_r = vb_r = None
    ro, rl = orc.decode_partials(q64, k64, v64, w, G, S, scale, Kbar=kb_r, Vbar=vb_r)
    empty = ~np.isfinite(rl)
    assert (np.isneginf(pl) == empty).all()
    assert (po[empty] == 0).all()
    if (~empty).any():
        assert_close(po[~empty], pl[~empty], ro[~empty], rl[~empty], TOL_BF16, "decode chunks")


@pytest.mark.parametrize("schedule", ["split", "fused"])
def test_decode_equals_prefill_last_row(schedule):
    print(f"[case] decode {schedule} vs prefill row", flush=True)
    B, Hq, Hkv, n, d, w, G = 2, 8, 2, 2048, 128, 200, 16
    Q = rand((B, Hq, n, d), 12, torch.bfloat16)
    K = rand((B, Hkv, n, d), 13, torch.bfloat16)
    V = rand((B, Hkv, n, d), 14, torch.bfloat16)
    Kb, Vb = msa.msa_pool_landmarks(K, V, G)
    O, L = msa.msa_attn_fwd(Q, K, V, Kb, Vb, w, G, out_dtype=torch.float32)
    q = Q[:, :, -1].contiguous()
    for S in (1, 2, 5, 16):
        Od, Ld = msa.msa_decode_fwd(q, K, V, Kb, Vb, w, G, S, out_dtype=torch.float32, schedule=schedule)
        torch.cuda.synchronize()
        assert (Od - O[:, :, -1]).abs().max().item() < 2e-3
        assert (Ld - L[:, :, -1]).abs().max().item() < 1e-4


DEC_SEQS = (0, 9, 18, 27, 36, 45, 54, 63)


@pytest.fixture(scope="module")
def dec512k():
    """The 512K decode workload run once under both schedules (the fused one
    is what the library picks and bench.py times); inputs stay on the GPU."""
    cfg = wl.DECODE_512K
    print(f"[case] {cfg.name} (fixture)", flush=True)
    q, Kc, Vc = wl.device_decode_inputs(cfg, dev())
    Kb, Vb = msa.msa_pool_landmarks(Kc, Vc, cfg.num_landmarks)
    desc = msa.decode_desc(cfg.batch, cfg.heads_q, cfg.heads_kv, cfg.ctx_len, cfg.head_dim, cfg.window,
                           cfg.num_landmarks, cfg.num_splits, cfg.scale, msa.MSA_DTYPE_BF16, msa.MSA_DTYPE_F32)
    ws = torch.empty(msa.msa_decode_workspace_size(desc) // 4, dtype=torch.float32, device=dev())
    args = (q, Kc, Vc, Kb, Vb, cfg.window, cfg.num_landmarks, cfg.num_splits, cfg.scale)
    r = {"cfg": cfg, "q": q, "Kc": Kc, "Vc": Vc}
    r["O32"], r["L32"] = msa.msa_decode_fwd(*args, out_dtype=torch.float32)
    r["O16"], _ = msa.msa_decode_fwd(*args)
    r["Os"], r["Ls"] = msa.msa_decode_fwd(*args, out_dtype=torch.float32, workspace=ws, schedule="split")
    po, pl = msa.decode_partials(ws, cfg.num_splits, cfg.batch, cfg.heads_q, cfg.head_dim)
    r["po"], r["pl"] = host64(po[:, 0]), host64(pl[:, 0])
    # the same caches holding sequences of different lengths (incremental decode)
    r["lens"] = wl.decode_lengths(cfg.batch, cfg.ctx_len)
    lens_d = torch.from_numpy(r["lens"]).to(dev())
    r["Ov"], r["Lv"] = msa.msa_decode_fwd_varlen(q, Kc, Vc, Kb, Vb, lens_d, *args[5:], out_dtype=torch.float32)
    r["Ovs"], r["Lvs"] = msa.msa_decode_fwd_varlen(q, Kc, Vc, Kb, Vb, lens_d, *args[5:], out_dtype=torch.float32,
                                                   workspace=ws, schedule="split")
    torch.cuda.synchronize()
    del Kb, Vb, ws
    yield r
    r.clear()
    torch.cuda.empty_cache()


def test_decode_workload_512k_store(dec512k):
    assert torch.equal(dec512k["O16"], bf16_rne(dec512k["O32"]))


@pytest.mark.parametrize("b", DEC_SEQS)
def test_decode_workload_512k(dec512k, b):
    r = dec512k
    cfg = r["cfg"]
    print(f"[case] {cfg.name} seq {b}", flush=True)
    k64, v64 = host64(r["Kc"][b:b + 1]), host64(r["Vc"][b:b + 1])
    q64 = host64(r["q"][b:b + 1])
    o_ref, l_ref = orc.decode(q64, k64, v64, cfg.window, cfg.num_landmarks, cfg.scale)
    assert_close(host64(r["O32"][b:b + 1]), host64(r["L32"][b:b + 1]), o_ref, l_ref, TOL_BF16,
                 f"{cfg.name} seq {b} (64 heads)")
    assert_close(host64(r["Os"][b:b + 1]), host64(r["Ls"][b:b + 1]), o_ref, l_ref, TOL_BF16,
                 f"{cfg.name} seq {b} (64 heads), split schedule")
    n = int(r["lens"][b])
    L = cfg.ctx_len // cfg.num_landmarks
    ov, lv = orc.decode_varlen(q64, k64, v64, [n], cfg.window, L, cfg.num_landmarks, cfg.scale)
    for key, sched in (("", "fused"), ("s", "split")):
        assert_close(host64(r["Ov" + key][b:b + 1]), host64(r["Lv" + key][b:b + 1]), ov, lv, TOL_BF16,
                     f"{cfg.name} seq {b} at length {n} (64 heads), {sched} schedule")
    if b == 0:
        kb_r = host64(torch.from_numpy(orc.pool(k64, cfg.num_landmarks)).to(torch.bfloat16))
        vb_r = host64(torch.from_numpy(orc.pool(v64, cfg.num_landmarks)).to(torch.bfloat16))
        ro, rl = orc.decode_partials(q64, k64, v64, cfg.window, cfg.num_landmarks, cfg.num_splits,
                                     cfg.scale, Kbar=kb_r, Vbar=vb_r)
        assert_close(r["po"], r["pl"], ro[:, 0], rl[:, 0], TOL_BF16, f"{cfg.name} seq 0 chunk partials")
