"""GPU parity on seeded random small shapes: batch, GQA group, head dim,
sequence length (ragged against the 128-row and 64-key tiles), landmark
count (0 or a divisor of n) and window (1 to beyond n) drawn from a fixed
seed, each case compared on every row with the fp64 oracle: the prefill's
float32 epilogue within the bf16 bounds and its bf16 store exactly RNE of
it; the backward within BWD_TOL; decode under both schedules."""
import math

import numpy as np
import pytest
import torch

from oracle import msa_oracle as orc
from tests.gpu_util import TOL_BF16, assert_close, bf16_rne, dev, host64
from tests.test_gpu_backward import BWD_TOL, grade, oracle_forward

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


def _shapes(count, seed, n_max):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        B = int(rng.integers(1, 3))
        Hkv = int(rng.choice([1, 2, 4]))
        Hq = Hkv * int(rng.choice([1, 2, 4, 8]))
        d = int(rng.choice([64, 128]))
        G = int(rng.integers(0, 12))
        if G:
            n = G * int(rng.integers(1, max(2, n_max // G)))
        else:
            n = int(rng.integers(1, n_max))
        if n < 1 or n > n_max:
            continue
        w = int(rng.choice([1, 2, 63, 64, 65, int(rng.integers(1, n + 1)), n + 5]))
        out.append((B, Hq, Hkv, n, d, w, G))
    return out


def _rand(shape, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32).to(torch.bfloat16).to(dev())


@pytest.mark.parametrize("B,Hq,Hkv,n,d,w,G", _shapes(14, 21, 900))
def test_attn_random_bf16(B, Hq, Hkv, n, d, w, G):
    print(f"[case] random attn B={B} Hq={Hq} Hkv={Hkv} n={n} d={d} w={w} G={G}", flush=True)
    Q, K, V = _rand((B, Hq, n, d), 31), _rand((B, Hkv, n, d), 32), _rand((B, Hkv, n, d), 33)
    scale = 1.0 / math.sqrt(d)
    Kb, Vb = msa.msa_pool_landmarks(K, V, G) if G else (None, None)
    O32, L32 = msa.msa_attn_fwd(Q, K, V, Kb, Vb, w, G, scale, out_dtype=torch.float32)
    O16, L16 = msa.msa_attn_fwd(Q, K, V, Kb, Vb, w, G, scale)
    torch.cuda.synchronize()
    o_ref, l_ref = orc.attn_dense(host64(Q), host64(K), host64(V), w, G, scale)
    assert_close(host64(O32), host64(L32), o_ref, l_ref, TOL_BF16, f"random n={n} w={w} G={G} d={d}")
    assert torch.equal(O16, bf16_rne(O32))
    assert torch.equal(L16, L32)


@pytest.mark.parametrize("B,Hq,Hkv,n,d,w,G", _shapes(6, 22, 500))
def test_bwd_random(B, Hq, Hkv, n, d, w, G):
    print(f"[case] random bwd B={B} Hq={Hq} Hkv={Hkv} n={n} d={d} w={w} G={G}", flush=True)
    Q, K, V = _rand((B, Hq, n, d), 41), _rand((B, Hkv, n, d), 42), _rand((B, Hkv, n, d), 43)
    dO = _rand((B, Hq, n, d), 44)
    scale = 1.0 / math.sqrt(d)
    O_in, LSE_in, O_ref = oracle_forward(Q, K, V, w, G, scale)
    Kb, Vb = msa.msa_pool_landmarks(K, V, G) if G else (None, None)
    dQ, dK, dV = msa.msa_attn_bwd(Q, K, V, Kb, Vb, O_in, LSE_in, dO, w, G, scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    q64, k64, v64, do64 = host64(Q), host64(K), host64(V), host64(dO)
    ref = orc.attn_bwd(q64, k64, v64, do64, w, G, scale, O=O_ref)
    # When every row sees only itself, P = 1 and D = dP, so dS and with it
    # the exact dQ and dK are zero: the kernel's values are the float32
    # rounding of dP - D, whose terms are as large as |dO_i| |V_i|.  Bound
    # them by 2^-16 of the largest such product times scale and max |K|, |Q|.
    cancel = scale * np.linalg.norm(do64, axis=-1).max() * np.linalg.norm(v64, axis=-1).max() * \
        max(np.abs(k64).max(), np.abs(q64).max())
    for name, got, r in zip(("dQ", "dK", "dV"), (dQ, dK, dV), ref):
        what = f"random {name} n={n} w={w} G={G} d={d}"
        if not np.any(r):
            err = float(np.abs(host64(got)).max())
            print(f"[parity] {what}: exact gradient 0, max |d| {err:.3e} (bound {2.0 ** -16 * cancel:.3e})", flush=True)
            assert err <= 2.0 ** -16 * cancel, what
        else:
            grade(host64(got), r, what, BWD_TOL)


@pytest.mark.parametrize("schedule", ["split", "fused"])
@pytest.mark.parametrize("B,Hq,Hkv,ctx,d,w,G", _shapes(6, 23, 3000))
def test_decode_random(B, Hq, Hkv, ctx, d, w, G, schedule):
    S = int(np.random.default_rng(ctx * 7 + w).integers(1, 20))
    print(f"[case] random decode {schedule} B={B} Hq={Hq} Hkv={Hkv} ctx={ctx} d={d} w={w} G={G} S={S}", flush=True)
    q, Kc, Vc = _rand((B, Hq, d), 51), _rand((B, Hkv, ctx, d), 52), _rand((B, Hkv, ctx, d), 53)
    scale = 1.0 / math.sqrt(d)
    Kb, Vb = msa.msa_pool_landmarks(Kc, Vc, G) if G else (None, None)
    O32, L32 = msa.msa_decode_fwd(q, Kc, Vc, Kb, Vb, w, G, S, scale, out_dtype=torch.float32, schedule=schedule)
    O16, _ = msa.msa_decode_fwd(q, Kc, Vc, Kb, Vb, w, G, S, scale, schedule=schedule)
    torch.cuda.synchronize()
    o_ref, l_ref = orc.decode(host64(q), host64(Kc), host64(Vc), w, G, scale)
    assert_close(host64(O32), host64(L32), o_ref, l_ref, TOL_BF16, f"random decode ctx={ctx} w={w} G={G} S={S}")
    assert torch.equal(O16, bf16_rne(O32))
