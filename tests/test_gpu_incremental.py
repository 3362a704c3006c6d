"""GPU parity of incremental decode: msa_decode_fwd_varlen on sequences of
different lengths in one cache and msa_append_kv growing them token by
token, through the C ABI, against the fp64 oracle on the same seeded
inputs.  Cache rows at or past a sequence's length hold large values, so a
kernel that read them would fail the comparison."""
import math

import numpy as np
import pytest
import torch

from oracle import msa_oracle as orc
from tests.gpu_util import TOL_BF16, assert_close, bf16_rne, dev, host64

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


def rand(shape, seed, dtype=torch.bfloat16):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32).to(dtype).to(dev())


def poison_tail(Kc, Vc, lens):
    """Rows at or past each length: K scaled by 40, V set to 1000."""
    for b, n in enumerate(lens):
        Kc[b, :, n:] *= 40
        Vc[b, :, n:] = 1000.0


def rounded_prefix_landmarks(k64, lens, L, G):
    """Oracle landmarks of each sequence's own prefix, rounded to bf16 (what
    the library stores), [B][Hkv][G][d] float64."""
    out = np.zeros(k64.shape[:2] + (G, k64.shape[-1]))
    for b, n in enumerate(lens):
        lm = orc.pool_prefix(k64[b:b + 1], n, L, G)[0]
        out[b] = host64(torch.from_numpy(lm).to(torch.bfloat16))
    return out


VARLEN = [
    # B, Hq, Hkv, C, d, w, G, S, lens
    (6, 8, 2, 2048, 128, 100, 32, 8, [2048, 1, 0, 777, 64, 1500]),
    (4, 16, 1, 1024, 64, 37, 64, 40, [1024, 1000, 16, 17]),       # more chunks than entries allow
    (3, 4, 4, 512, 128, 1000, 0, 3, [300, 512, 2]),                 # window covers everything, no landmarks
    (5, 8, 8, 4096, 128, 300, 16, 7, [4096, 4095, 257, 3000, 1]),
    (2, 6, 2, 2048, 128, 129, 32, 1, [1111, 2048]),                 # unsplit
]


@pytest.mark.parametrize("schedule", ["split", "fused"])
@pytest.mark.parametrize("B,Hq,Hkv,C,d,w,G,S,lens", VARLEN)
def test_decode_varlen_small(B, Hq, Hkv, C, d, w, G, S, lens, schedule):
    print(f"[case] decode_varlen {schedule} B={B} Hq={Hq} Hkv={Hkv} C={C} d={d} w={w} G={G} S={S} "
          f"lens={lens}", flush=True)
    q = rand((B, Hq, d), 21)
    Kc, Vc = rand((B, Hkv, C, d), 22), rand((B, Hkv, C, d), 23)
    poison_tail(Kc, Vc, lens)
    scale = 1.0 / math.sqrt(d)
    Kb, Vb = msa.msa_pool_landmarks(Kc, Vc, G) if G else (None, None)  # slots of incomplete blocks: poisoned
    lens_d = torch.tensor(lens, dtype=torch.int32, device=dev())
    desc = msa.decode_desc(B, Hq, Hkv, C, d, w, G, S, scale, msa.MSA_DTYPE_BF16, msa.MSA_DTYPE_F32)
    ws = torch.empty(msa.msa_decode_workspace_size(desc) // 4, dtype=torch.float32, device=dev())
    O32, L32 = msa.msa_decode_fwd_varlen(q, Kc, Vc, Kb, Vb, lens_d, w, G, S, scale, out_dtype=torch.float32,
                                         workspace=ws, schedule=schedule)
    po, pl = msa.decode_partials(ws, S, B, Hq, d)
    po, pl = host64(po), host64(pl)
    O16, _ = msa.msa_decode_fwd_varlen(q, Kc, Vc, Kb, Vb, lens_d, w, G, S, scale, schedule=schedule)
    torch.cuda.synchronize()
    L = C // G if G else 1
    q64, k64, v64 = host64(q), host64(Kc), host64(Vc)
    o_ref, l_ref = orc.decode_varlen(q64, k64, v64, lens, w, L, G, scale)
    live = np.array(lens) > 0
    assert_close(host64(O32)[live], host64(L32)[live], o_ref[live], l_ref[live], TOL_BF16, "decode_varlen")
    if (~live).any():  # an empty sequence: O = 0, LSE = -inf
        assert (host64(O32)[~live] == 0).all() and np.isneginf(host64(L32)[~live]).all()
    assert torch.equal(O16, bf16_rne(O32))
    if schedule != "split":
        return
    kb_r = rounded_prefix_landmarks(k64, lens, L, G) if G else None
    vb_r = rounded_prefix_landmarks(v64, lens, L, G) if G else None
    ro, rl = orc.decode_varlen_partials(q64, k64, v64, lens, w, L, G, S, scale, Kbar=kb_r, Vbar=vb_r)
    empty = ~np.isfinite(rl)
    assert (np.isneginf(pl) == empty).all()
    assert (po[empty] == 0).all()
    assert_close(po[~empty], pl[~empty], ro[~empty], rl[~empty], TOL_BF16, "decode_varlen chunks")


@pytest.mark.parametrize("schedule", ["split", "fused"])
def test_decode_varlen_full_lengths_equal_static(schedule):
    print(f"[case] decode_varlen {schedule} full lengths vs static", flush=True)
    B, Hq, Hkv, C, d, w, G, S = 4, 8, 2, 4096, 128, 200, 64, 8
    q = rand((B, Hq, d), 31)
    Kc, Vc = rand((B, Hkv, C, d), 32), rand((B, Hkv, C, d), 33)
    Kb, Vb = msa.msa_pool_landmarks(Kc, Vc, G)
    lens_d = torch.full((B,), C, dtype=torch.int32, device=dev())
    Ov, Lv = msa.msa_decode_fwd_varlen(q, Kc, Vc, Kb, Vb, lens_d, w, G, S, out_dtype=torch.float32, schedule=schedule)
    Os, Ls = msa.msa_decode_fwd(q, Kc, Vc, Kb, Vb, w, G, S, out_dtype=torch.float32, schedule=schedule)
    torch.cuda.synchronize()
    assert torch.equal(Ov, Os) and torch.equal(Lv, Ls)


def test_decode_varlen_clamps_lengths():
    # lengths outside [0, C] are clamped on the device: -5 acts as 0, C + 100 as C
    print("[case] decode_varlen clamped lengths", flush=True)
    B, Hq, Hkv, C, d, w, G, S = 3, 4, 1, 1024, 128, 64, 16, 4
    q = rand((B, Hq, d), 41)
    Kc, Vc = rand((B, Hkv, C, d), 42), rand((B, Hkv, C, d), 43)
    Kb, Vb = msa.msa_pool_landmarks(Kc, Vc, G)
    bad = torch.tensor([-5, C + 100, 500], dtype=torch.int32, device=dev())
    good = torch.tensor([0, C, 500], dtype=torch.int32, device=dev())
    Ob, Lb = msa.msa_decode_fwd_varlen(q, Kc, Vc, Kb, Vb, bad, w, G, S, out_dtype=torch.float32)
    Og, Lg = msa.msa_decode_fwd_varlen(q, Kc, Vc, Kb, Vb, good, w, G, S, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(Ob, Og) and torch.equal(Lb, Lg)


# ------------------------------------------------------------------ append

@pytest.mark.parametrize("schedule", ["split", "fused"])
@pytest.mark.parametrize("d", [128, 64])
def test_append_then_decode(d, schedule):
    """Grow four sequences token by token (one idle), decoding after every
    append; each step is graded against the oracle's decode of the same
    prefix, and the landmarks kept by the appends must equal, bit for bit,
    pooling the final cache."""
    B, Hq, Hkv, C, w, G, S, steps = 4, 8, 2, 1024, 40, 64, 6, 48
    L = C // G
    print(f"[case] append+decode {schedule} d={d} B={B} C={C} L={L} steps={steps}", flush=True)
    start = [0, 100, 990, 31]       # sequence 1 stays idle; sequence 2 runs past the capacity
    idle = [False, True, False, False]
    Kc, Vc = rand((B, Hkv, C, d), 51), rand((B, Hkv, C, d), 52)
    poison_tail(Kc, Vc, start)
    Kb, Vb = msa.msa_pool_landmarks(Kc, Vc, G)   # slots of blocks past each start: poisoned
    k_new, v_new = rand((steps, B, Hkv, d), 53), rand((steps, B, Hkv, d), 54)
    qs = rand((steps, B, Hq, d), 55)
    scale = 1.0 / math.sqrt(d)
    lens = list(start)
    k_ref, v_ref = host64(Kc), host64(Vc)
    for t in range(steps):
        pos = [-1 if idle[b] else lens[b] for b in range(B)]
        pos_d = torch.tensor(pos, dtype=torch.int32, device=dev())
        msa.msa_append_kv(k_new[t], v_new[t], pos_d, Kc, Vc, Kb, Vb, G)
        for b in range(B):
            if 0 <= pos[b] < C:
                lens[b] = pos[b] + 1
                k_ref[b, :, pos[b]] = host64(k_new[t, b])
                v_ref[b, :, pos[b]] = host64(v_new[t, b])
        lens_d = torch.tensor(lens, dtype=torch.int32, device=dev())
        O, LSE = msa.msa_decode_fwd_varlen(qs[t], Kc, Vc, Kb, Vb, lens_d, w, G, S, scale,
                                           out_dtype=torch.float32, schedule=schedule)
        torch.cuda.synchronize()
        live = [b for b in range(B) if lens[b] > 0]
        o_ref, l_ref = orc.decode_varlen(host64(qs[t])[live], k_ref[live], v_ref[live],
                                         [lens[b] for b in live], w, L, G, scale)
        assert_close(host64(O)[live], host64(LSE)[live], o_ref, l_ref, TOL_BF16, f"step {t} lens={lens}")
    # every row the appends wrote, and nothing else
    np.testing.assert_array_equal(host64(Kc), k_ref)
    np.testing.assert_array_equal(host64(Vc), v_ref)
    # landmarks of complete blocks: the same bits as pooling the final cache
    Kp, Vp = msa.msa_pool_landmarks(Kc, Vc, G)
    torch.cuda.synchronize()
    for b in range(B):
        done = lens[b] // L
        assert torch.equal(Kb[b, :, :done], Kp[b, :, :done]), b
        assert torch.equal(Vb[b, :, :done], Vp[b, :, :done]), b
    # every complete block holds the bf16 rounding of its exact mean
    for b in range(B):
        for blk in range(lens[b] // L):
            exact = k_ref[b, :, blk * L:(blk + 1) * L].mean(axis=1)
            np.testing.assert_allclose(host64(Kb[b, :, blk]), exact, atol=2 ** -8 * np.abs(exact).max() + 1e-6)


# ------------------------------------------------------------------ paged caches

def to_pages(Kc, Vc, page, seed, extra=3):
    """Scatter contiguous caches [B][Hkv][C][d] into page pools under a
    seeded random permutation; `extra` pool pages are unused and hold large
    values.  Returns (Kpages, Vpages, table int32 [B][C/page] on the device,
    table as numpy)."""
    B, Hkv, C, d = Kc.shape
    P = C // page
    n_pages = B * P + extra
    perm = np.random.default_rng(seed).permutation(n_pages)[:B * P].reshape(B, P).astype(np.int32)
    Kp = rand((n_pages, Hkv, page, d), seed) * 50
    Vp = rand((n_pages, Hkv, page, d), seed + 1) * 50
    for b in range(B):
        for lp in range(P):
            Kp[int(perm[b, lp])] = Kc[b, :, lp * page:(lp + 1) * page]
            Vp[int(perm[b, lp])] = Vc[b, :, lp * page:(lp + 1) * page]
    return Kp, Vp, torch.from_numpy(perm).to(dev()), perm


@pytest.mark.parametrize("schedule", ["split", "fused"])
@pytest.mark.parametrize("page", [32, 64, 256])
def test_paged_decode_equals_contiguous(page, schedule):
    B, Hq, Hkv, C, d, w, G, S, lens = VARLEN[0]
    print(f"[case] paged decode {schedule} page={page} B={B} C={C} lens={lens}", flush=True)
    q = rand((B, Hq, d), 61)
    Kc, Vc = rand((B, Hkv, C, d), 62), rand((B, Hkv, C, d), 63)
    poison_tail(Kc, Vc, lens)
    Kb, Vb = msa.msa_pool_landmarks(Kc, Vc, G)
    lens_d = torch.tensor(lens, dtype=torch.int32, device=dev())
    Kp, Vp, table, perm = to_pages(Kc, Vc, page, 64 + page)
    scale = 1.0 / math.sqrt(d)
    Oc, Lc = msa.msa_decode_fwd_varlen(q, Kc, Vc, Kb, Vb, lens_d, w, G, S, scale, out_dtype=torch.float32, schedule=schedule)
    Op, Lp = msa.msa_decode_fwd_paged(q, Kp, Vp, table, Kb, Vb, lens_d, w, G, S, scale, out_dtype=torch.float32, schedule=schedule)
    torch.cuda.synchronize()
    # same rows, same tiles, same order: the same bits
    assert torch.equal(Op, Oc) and torch.equal(Lp, Lc)
    # pages past each sequence's length are never looked up: unmapping them
    # (id -1) changes nothing
    cut = table.clone()
    for b, n in enumerate(lens):
        cut[b, -(-n // page):] = -1
    Ou, Lu = msa.msa_decode_fwd_paged(q, Kp, Vp, cut, Kb, Vb, lens_d, w, G, S, scale, out_dtype=torch.float32,
                                      schedule=schedule)
    torch.cuda.synchronize()
    assert torch.equal(Ou, Oc) and torch.equal(Lu, Lc)
    # and against the oracle over the gathered pools
    k64 = orc.gather_pages(host64(Kp), perm, page)
    v64 = orc.gather_pages(host64(Vp), perm, page)
    o_ref, l_ref = orc.decode_varlen(host64(q), k64, v64, lens, w, C // G, G, scale)
    live = np.array(lens) > 0
    assert_close(host64(Op)[live], host64(Lp)[live], o_ref[live], l_ref[live], TOL_BF16, f"paged page={page}")


@pytest.mark.parametrize("schedule", ["split", "fused"])
def test_paged_append_then_decode_equals_contiguous(schedule):
    """The append + decode sequence of test_append_then_decode on paged caches
    gives the bits of the contiguous run at every step."""
    B, Hq, Hkv, C, d, w, G, S, steps, page = 4, 8, 2, 1024, 128, 40, 64, 6, 40, 32
    L = C // G
    print(f"[case] paged append+decode {schedule} page={page} steps={steps}", flush=True)
    start = [0, 100, 1000, 31]
    idle = [False, True, False, False]
    Kc, Vc = rand((B, Hkv, C, d), 71), rand((B, Hkv, C, d), 72)
    poison_tail(Kc, Vc, start)
    Kb, Vb = msa.msa_pool_landmarks(Kc, Vc, G)
    Kp, Vp, table, perm = to_pages(Kc, Vc, page, 73)
    Kbp, Vbp = Kb.clone(), Vb.clone()
    k_new, v_new = rand((steps, B, Hkv, d), 74), rand((steps, B, Hkv, d), 75)
    qs = rand((steps, B, Hq, d), 76)
    lens = list(start)
    for t in range(steps):
        pos = torch.tensor([-1 if idle[b] else lens[b] for b in range(B)], dtype=torch.int32, device=dev())
        msa.msa_append_kv(k_new[t], v_new[t], pos, Kc, Vc, Kb, Vb, G)
        msa.msa_append_kv_paged(k_new[t], v_new[t], pos, Kp, Vp, table, Kbp, Vbp, G)
        lens = [min(C, lens[b] + 1) if not idle[b] else lens[b] for b in range(B)]
        lens_d = torch.tensor(lens, dtype=torch.int32, device=dev())
        Oc, Lc = msa.msa_decode_fwd_varlen(qs[t], Kc, Vc, Kb, Vb, lens_d, w, G, S, out_dtype=torch.float32, schedule=schedule)
        Op, Lp = msa.msa_decode_fwd_paged(qs[t], Kp, Vp, table, Kbp, Vbp, lens_d, w, G, S, out_dtype=torch.float32, schedule=schedule)
        torch.cuda.synchronize()
        assert torch.equal(Op, Oc) and torch.equal(Lp, Lc), t
    assert torch.equal(Kbp, Kb) and torch.equal(Vbp, Vb)
    # every row the paged appends wrote sits where the table says
    gathered = orc.gather_pages(host64(Kp), perm, page)
    np.testing.assert_array_equal(gathered, host64(Kc))
    gathered = orc.gather_pages(host64(Vp), perm, page)
    np.testing.assert_array_equal(gathered, host64(Vc))


@pytest.mark.parametrize("schedule", ["split", "fused"])
def test_paged_decode_64k(schedule):
    """A 64K-token capacity with the full window and 1024-row landmark blocks:
    paged (64-row pages, random permutation) equals contiguous bit for bit,
    and two sequences are graded against the oracle."""
    B, Hq, Hkv, C, d, w, G, S, page = 4, 32, 4, 65536, 128, 4096, 64, 16, 64
    print(f"[case] paged decode 64k {schedule}", flush=True)
    lens = [int(x) for x in np.random.default_rng(90).integers(C // 2, C + 1, size=B)]
    q = rand((B, Hq, d), 91)
    Kc, Vc = rand((B, Hkv, C, d), 92), rand((B, Hkv, C, d), 93)
    poison_tail(Kc, Vc, lens)
    Kb, Vb = msa.msa_pool_landmarks(Kc, Vc, G)
    lens_d = torch.tensor(lens, dtype=torch.int32, device=dev())
    Kp, Vp, table, perm = to_pages(Kc, Vc, page, 94)
    scale = 1.0 / math.sqrt(d)
    Oc, Lc = msa.msa_decode_fwd_varlen(q, Kc, Vc, Kb, Vb, lens_d, w, G, S, scale, out_dtype=torch.float32, schedule=schedule)
    Op, Lp = msa.msa_decode_fwd_paged(q, Kp, Vp, table, Kb, Vb, lens_d, w, G, S, scale, out_dtype=torch.float32, schedule=schedule)
    torch.cuda.synchronize()
    assert torch.equal(Op, Oc) and torch.equal(Lp, Lc)
    for b in (0, 3):
        o_ref, l_ref = orc.decode_varlen(host64(q[b:b + 1]), host64(Kc[b:b + 1]), host64(Vc[b:b + 1]), [lens[b]],
                                         w, C // G, G, scale)
        assert_close(host64(Op[b:b + 1]), host64(Lp[b:b + 1]), o_ref, l_ref, TOL_BF16, f"paged 64k seq {b}")
