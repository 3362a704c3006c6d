"""GPU parity of the backward (msa_attn_bwd) through the C ABI against the
fp64 oracle's chain rule on the same seeded inputs: dQ, dK, dV with float32
outputs graded element by element (every element on the small cases; whole
KV groups, each KV head with its query heads, on the 32K workload and on the
128K GQA workload that bench.py times, plus sampled dQ rows of other heads);
the bf16 outputs must equal the round-to-nearest-even of the float32 ones.

The backward's inputs include the forward's output O and LSE.  Both sides
are handed the same ones, from the oracle's forward: O rounded to bf16 (as a
training step stores it) and LSE in float32.  The oracle's backward takes
that O for the softmax term D = rowsum(dO * O), as the kernel does, so the
comparison measures the kernel's own arithmetic, not the rounding of its
inputs.  Bound: the gradients are sums of products whose factors (P, dS
and the bf16 inputs) enter the matrix cores as bf16 with float32
accumulation, so each element errs by a few bf16 roundings of its largest
terms; the test bounds the error by a fraction of the RMS of the element's
row and tensor (see BWD_TOL).  The GPU forward feeding the GPU backward is
covered end to end by the determinism and bf16 checks and by smoke()."""
import math

import numpy as np
import pytest
import torch

import msa_inputs as wl
from oracle import msa_oracle as orc
from tests.gpu_util import bf16_rne, dev, host64

pytestmark = pytest.mark.gpu

msa = pytest.importorskip("long_context_sparse_msa_amd")

# Per element: |dX - ref| <= max_row * (rms of ref's row + floor * rms of ref)
# (a gradient row's terms share one scale; the floor covers rows whose
# exact gradient is 0, such as dQ of row 0, which sees only itself);
# over the tensor: mean |dX - ref| <= mean_rms * rms(ref).  With both sides
# handed the same O, an element errs by bf16 roundings (2^-9 relative) of
# the P and dS factors of its terms, accumulated in float32: max_row = 0.03
# is about fifteen such roundings of the row's scale (measured worst 0.0135
# over every element of two whole KV groups at 128K; typical 0.007).
BWD_TOL = dict(max_row=0.03, floor=0.05, mean_rms=3e-3)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    msa.lib()  # a missing library is an error, not a skip
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def rand(shape, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32).to(torch.bfloat16).to(dev())


def grade(got, ref, what, tol=BWD_TOL):
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    rms = float(np.sqrt((ref ** 2).mean()))
    if rms == 0.0:
        assert err.max() <= 1e-6, what
        return
    row_rms = np.sqrt((ref ** 2).mean(axis=-1, keepdims=True))
    rel = err / (row_rms + tol["floor"] * rms)
    stats = dict(max_row=float(rel.max()), mean_rms=float(err.mean()) / rms)
    print(f"[parity] {what}: max |d|/(row rms + {tol['floor']} rms)={stats['max_row']:.3e} "
          f"(p99.99 {float(np.quantile(rel, 0.9999)):.3e}), mean|d|/rms={stats['mean_rms']:.3e}, "
          f"rms={rms:.3e}", flush=True)
    assert stats["max_row"] <= tol["max_row"], (what, stats)
    assert stats["mean_rms"] <= tol["mean_rms"], (what, stats)


def run_fwd_bwd(Q, K, V, dO, w, G, scale, out_dtype=torch.float32):
    """GPU forward, then the GPU backward handed its O and LSE."""
    Kb, Vb = msa.msa_pool_landmarks(K, V, G) if G else (None, None)
    O, LSE = msa.msa_attn_fwd(Q, K, V, Kb, Vb, w, G, scale)
    return msa.msa_attn_bwd(Q, K, V, Kb, Vb, O, LSE, dO, w, G, scale, out_dtype=out_dtype), (Kb, Vb, O, LSE)


def oracle_forward(Q, K, V, w, G, scale):
    """The forward output and LSE to hand to both backwards, from the fp64
    oracle: (O bf16 on the device, LSE float32 on the device, the same bf16
    O in fp64 for the oracle)."""
    o, lse = orc.attn_dense(host64(Q), host64(K), host64(V), w, G, scale)
    o16 = torch.from_numpy(o).float().to(torch.bfloat16)
    return o16.to(dev()), torch.from_numpy(lse).float().to(dev()), o16.double().numpy()


SMALL = [
    # B, Hq, Hkv, n, d, w, G
    (1, 2, 1, 256, 128, 64, 4),
    (2, 8, 2, 512, 128, 100, 8),
    (1, 4, 2, 300, 128, 37, 3),       # ragged tail (L = 100)
    (1, 4, 4, 1024, 64, 200, 16),
    (1, 2, 2, 384, 128, 1000, 0),     # window covers the sequence, no landmarks
    (1, 2, 1, 256, 128, 16, 256),     # one-token landmarks
    (1, 16, 1, 640, 128, 129, 5),     # 16 query heads per KV head
    (1, 1, 1, 1, 128, 1, 1),          # a single token
]


@pytest.mark.parametrize("B,Hq,Hkv,n,d,w,G", SMALL)
def test_bwd_small(B, Hq, Hkv, n, d, w, G):
    print(f"[case] bwd B={B} Hq={Hq} Hkv={Hkv} n={n} d={d} w={w} G={G}", flush=True)
    Q, K, V = rand((B, Hq, n, d), 1), rand((B, Hkv, n, d), 2), rand((B, Hkv, n, d), 3)
    dO = rand((B, Hq, n, d), 4)
    scale = 1.0 / math.sqrt(d)
    O_in, LSE_in, O_ref = oracle_forward(Q, K, V, w, G, scale)
    Kb, Vb = msa.msa_pool_landmarks(K, V, G) if G else (None, None)
    dQ, dK, dV = msa.msa_attn_bwd(Q, K, V, Kb, Vb, O_in, LSE_in, dO, w, G, scale, out_dtype=torch.float32)
    dQ16, dK16, dV16 = msa.msa_attn_bwd(Q, K, V, Kb, Vb, O_in, LSE_in, dO, w, G, scale, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = orc.attn_bwd(host64(Q), host64(K), host64(V), host64(dO), w, G, scale, O=O_ref)
    for name, got, r in zip(("dQ", "dK", "dV"), (dQ, dK, dV), ref):
        grade(host64(got), r, f"{name} n={n} w={w} G={G}")
    assert torch.equal(dQ16, bf16_rne(dQ)) and torch.equal(dK16, bf16_rne(dK)) and torch.equal(dV16, bf16_rne(dV))


def test_bwd_deterministic():
    print("[case] bwd repeat", flush=True)
    B, Hq, Hkv, n, d, w, G = 1, 8, 2, 2048, 128, 300, 16
    Q, K, V, dO = rand((B, Hq, n, d), 5), rand((B, Hkv, n, d), 6), rand((B, Hkv, n, d), 7), rand((B, Hq, n, d), 8)
    (a, b, c), fwd = run_fwd_bwd(Q, K, V, dO, w, G, 1 / math.sqrt(d))
    a2, b2, c2 = msa.msa_attn_bwd(Q, K, V, *fwd, dO, w, G, 1 / math.sqrt(d))
    torch.cuda.synchronize()
    assert torch.equal(a, a2) and torch.equal(b, b2) and torch.equal(c, c2)


@pytest.fixture(scope="module")
def bwd32k():
    """bf16_32k (8/8 heads, n 32768, w 4096, G 512; 32 landmark segments of 1024 rows)."""
    cfg = wl.BF16_32K
    print(f"[case] {cfg.name} backward (fixture)", flush=True)
    Q, K, V = wl.device_prefill_inputs(cfg, dev())
    dO = rand(tuple(Q.shape), 9)
    O_in, LSE_in, O_ref = oracle_forward(Q, K, V, cfg.window, cfg.num_landmarks, cfg.scale)
    Kb, Vb = msa.msa_pool_landmarks(K, V, cfg.num_landmarks)
    dQ, dK, dV = msa.msa_attn_bwd(Q, K, V, Kb, Vb, O_in, LSE_in, dO, cfg.window, cfg.num_landmarks, cfg.scale)
    torch.cuda.synchronize()
    yield cfg, Q, K, V, dO, O_ref, dQ, dK, dV
    torch.cuda.empty_cache()


@pytest.mark.parametrize("g", [0, 5])
def test_bwd_workload_32k_kv_head(bwd32k, g):
    cfg, Q, K, V, dO, O_ref, dQ, dK, dV = bwd32k
    print(f"[case] {cfg.name} backward kv head {g}", flush=True)
    sl = slice(g, g + 1)
    ref = orc.attn_bwd(host64(Q[:, sl]), host64(K[:, sl]), host64(V[:, sl]), host64(dO[:, sl]), cfg.window,
                       cfg.num_landmarks, cfg.scale, O=O_ref[:, sl])
    for name, got, r in zip(("dQ", "dK", "dV"), (dQ[:, sl], dK[:, sl], dV[:, sl]), ref):
        grade(host64(got), r, f"{cfg.name} {name} head {g}")


@pytest.fixture(scope="module")
def bwd128k():
    """gqa_128k (64/8 heads, n 131072, w 4096, G 512: 128 landmark segments,
    8 query heads summed into each KV head), as bench.py runs it: the GPU
    forward, then the backward with float32 and with bf16 gradients."""
    cfg = wl.GQA_128K
    print(f"[case] {cfg.name} backward (fixture)", flush=True)
    Q, K, V = wl.device_prefill_inputs(cfg, dev())
    dO = rand(tuple(Q.shape), 10)
    (dQ, dK, dV), fwd = run_fwd_bwd(Q, K, V, dO, cfg.window, cfg.num_landmarks, cfg.scale)
    g16 = msa.msa_attn_bwd(Q, K, V, *fwd, dO, cfg.window, cfg.num_landmarks, cfg.scale, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    yield cfg, Q, K, V, dO, fwd, (dQ, dK, dV), g16
    torch.cuda.empty_cache()


def test_bwd_workload_128k_bf16_is_rne(bwd128k):
    cfg, *_, g32, g16 = bwd128k
    for name, a, b in zip(("dQ", "dK", "dV"), g32, g16):
        assert torch.isfinite(a).all(), name
        assert torch.equal(b, bf16_rne(a)), name


def test_bwd_workload_128k_dq_rows(bwd128k):
    """dQ on 1024 sampled rows of heads 0, 9 and 63; those rows of O and
    LSE handed to the backward come from the oracle's forward."""
    cfg, Q, K, V, dO, (Kb, Vb, O, LSE), _, _ = bwd128k
    print(f"[case] {cfg.name} backward, sampled dQ rows", flush=True)
    L = cfg.seq_len // cfg.num_landmarks
    grp = cfg.heads_q // cfg.heads_kv
    O_in, LSE_in = O.clone(), LSE.clone()
    rows, o_ref = {}, {}
    for h in (0, 9, 63):
        g = h // grp
        rows[h] = np.sort(wl.sample_rows(cfg.seq_len, h, count=1024, window=cfg.window, block=L))
        ridx = torch.from_numpy(rows[h]).to(dev())
        Qr = np.zeros((1, 1, cfg.seq_len, cfg.head_dim))
        Qr[:, 0, rows[h]] = host64(Q[:, h].index_select(1, ridx))
        _, o, lse = orc.attn(Qr, host64(K[:, g:g + 1]), host64(V[:, g:g + 1]), cfg.window, cfg.num_landmarks,
                             cfg.scale, rows={0: rows[h]})[0]
        o16 = torch.from_numpy(o).float().to(torch.bfloat16)
        o_ref[h] = o16.double().numpy()
        O_in[:, h].index_copy_(1, ridx, o16.to(dev()))
        LSE_in[:, h].index_copy_(1, ridx, torch.from_numpy(lse).float().to(dev()))
    dQ, _, _ = msa.msa_attn_bwd(Q, K, V, Kb, Vb, O_in, LSE_in, dO, cfg.window, cfg.num_landmarks, cfg.scale)
    torch.cuda.synchronize()
    for h in rows:
        g = h // grp
        res = orc.attn_bwd_dq_rows(host64(Q[:, h:h + 1]), host64(K[:, g:g + 1]), host64(V[:, g:g + 1]),
                                   host64(dO[:, h:h + 1]), cfg.window, cfg.num_landmarks, cfg.scale,
                                   rows={0: rows[h]}, group_span=4096, O={0: o_ref[h]})
        r, ref = res[0]
        ridx = torch.from_numpy(r).to(dev())
        grade(host64(dQ[:, h].index_select(1, ridx)), ref, f"{cfg.name} dQ head {h} ({len(r)} rows)")


@pytest.mark.parametrize("g", [0, 7])
def test_bwd_workload_128k_kv_group(bwd128k, g):
    """Every element of dK and dV of KV head g, and of dQ of its 8 query
    heads: the window and landmark paths of the 8 heads summed per key, the
    128-segment landmark reduce, and the 1/L scatter, as bench.py runs them.
    The group's O and LSE handed to the backward come from the oracle."""
    cfg, Q, K, V, dO, (Kb, Vb, O, LSE), _, _ = bwd128k
    print(f"[case] {cfg.name} backward, KV group {g} in full", flush=True)
    grp = cfg.heads_q // cfg.heads_kv
    hs = slice(g * grp, (g + 1) * grp)
    ks = slice(g, g + 1)
    Qg, Kg, Vg = host64(Q[:, hs]), host64(K[:, ks]), host64(V[:, ks])
    o, lse = orc.attn_dense(Qg, Kg, Vg, cfg.window, cfg.num_landmarks, cfg.scale)
    o16 = torch.from_numpy(o).float().to(torch.bfloat16)
    del o
    O_in, LSE_in = O.clone(), LSE.clone()
    O_in[:, hs] = o16.to(dev())
    LSE_in[:, hs] = torch.from_numpy(lse).float().to(dev())
    dQ, dK, dV = msa.msa_attn_bwd(Q, K, V, Kb, Vb, O_in, LSE_in, dO, cfg.window, cfg.num_landmarks, cfg.scale)
    torch.cuda.synchronize()
    del O_in, LSE_in
    ref = orc.attn_bwd(Qg, Kg, Vg, host64(dO[:, hs]), cfg.window, cfg.num_landmarks, cfg.scale,
                       O=o16.double().numpy())
    for name, got, r in zip(("dQ", "dK", "dV"), (dQ[:, hs], dK[:, ks], dV[:, ks]), ref):
        grade(host64(got), r, f"{cfg.name} {name} KV group {g}")
