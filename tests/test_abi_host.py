"""Host-side tests of libmsa's C ABI: the library loads and exports every
symbol the header declares, validation rejects bad arguments before any
launch, and the schedule it reports is bit-exact against the oracle's
mask-derived plans.  No GPU is used (only host-only exports and calls that
fail validation)."""
import ctypes
import os
import re

import numpy as np
import pytest

import msa_inputs as wl
from oracle import msa_oracle as orc

msa = pytest.importorskip("long_context_sparse_msa_amd")
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    return msa.lib()


def header_functions():
    with open(os.path.join(ROOT, "include", "msa.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = header_functions()
    assert len(names) == 19
    assert sorted(msa.EXPORTS) == names
    for name in names:
        assert hasattr(L, name), name


def test_abi_version(L):
    assert msa.abi_version() == 3


def test_status_strings(L):
    for s in range(6):
        assert L.msa_status_string(s)
    assert L.msa_status_string(99) == b"unknown status"


def call_attn(desc, ptr=16):
    p = ctypes.c_void_p(ptr)
    return msa.lib().msa_attn_fwd(ctypes.byref(desc), p, p, p, p, p, p, None, None)


def base_desc(**kw):
    args = dict(batch=1, heads_q=4, heads_kv=2, seq_len=256, head_dim=128, window=64, num_landmarks=4,
                scale=0.1, in_dtype=msa.MSA_DTYPE_BF16, out_dtype=msa.MSA_DTYPE_BF16)
    args.update(kw)
    return msa.AttnDesc(*[args[k] for k, _ in msa.AttnDesc._fields_])


@pytest.mark.parametrize("kw,status", [
    (dict(window=0), 1), (dict(window=-3), 1), (dict(num_landmarks=-1), 1), (dict(num_landmarks=3), 1),
    (dict(heads_q=3), 1), (dict(heads_kv=0), 1), (dict(head_dim=96), 2), (dict(head_dim=256), 2),
    (dict(in_dtype=7), 1), (dict(out_dtype=5), 1), (dict(batch=-1), 1), (dict(seq_len=-5), 1),
    (dict(scale=float("nan")), 1), (dict(scale=float("inf")), 1), (dict(scale=0.0), 1), (dict(scale=-0.5), 1),
    (dict(in_dtype=msa.MSA_DTYPE_F32, out_dtype=msa.MSA_DTYPE_BF16), 2),
    (dict(seq_len=1 << 23), 2), (dict(seq_len=1 << 24, head_dim=64), 2),
])
def test_attn_validation(kw, status):
    assert call_attn(base_desc(**kw)) == status
    assert msa.lib().msa_last_error()


def test_attn_null_and_misaligned_pointers():
    L = msa.lib()
    d = base_desc()
    p = ctypes.c_void_p(16)
    assert L.msa_attn_fwd(ctypes.byref(d), None, p, p, p, p, p, None, None) == 1
    assert b"Q is NULL" in L.msa_last_error()
    assert L.msa_attn_fwd(ctypes.byref(d), p, p, p, ctypes.c_void_p(24), p, p, None, None) == 1
    assert b"Kbar is not 16-byte aligned" in L.msa_last_error()
    # no landmarks: Kbar/Vbar may be NULL; an empty problem launches nothing
    d0 = base_desc(num_landmarks=0, batch=0)
    assert L.msa_attn_fwd(ctypes.byref(d0), p, p, p, None, None, p, None, None) == 0


def test_python_binding_raises():
    with pytest.raises(msa.MsaError) as e:
        msa.msa_plan_rows(base_desc(window=0))
    assert e.value.status == 1


def dec_desc(**kw):
    args = dict(batch=2, heads_q=8, heads_kv=2, ctx_len=512, head_dim=128, window=64, num_landmarks=8,
                num_splits=4, scale=0.1, in_dtype=msa.MSA_DTYPE_BF16, out_dtype=msa.MSA_DTYPE_BF16, schedule=0)
    args.update(kw)
    return msa.DecodeDesc(*[args[k] for k, _ in msa.DecodeDesc._fields_])


@pytest.mark.parametrize("kw,status", [
    (dict(num_splits=0), 1), (dict(window=0), 1), (dict(num_landmarks=7), 1), (dict(ctx_len=0), 1),
    (dict(heads_q=6, heads_kv=4), 1), (dict(heads_q=64, heads_kv=2), 2), (dict(head_dim=32), 2),
    (dict(in_dtype=msa.MSA_DTYPE_F32), 2), (dict(ctx_len=1 << 23), 2), (dict(schedule=3), 1),
    (dict(schedule=-1), 1),
])
def test_decode_validation(kw, status):
    d = dec_desc(**kw)
    p = ctypes.c_void_p(16)
    assert msa.lib().msa_decode_fwd(ctypes.byref(d), p, p, p, p, p, p, 1 << 30, p, None, None) == status


def test_decode_workspace_checks():
    d = dec_desc()
    need = msa.msa_decode_workspace_size(d)
    assert need == 4 * 2 * 8 * 129 * 4
    p = ctypes.c_void_p(16)
    assert msa.lib().msa_decode_fwd(ctypes.byref(d), p, p, p, p, p, p, need - 4, p, None, None) == 3
    assert b"workspace" in msa.lib().msa_last_error()


def test_pool_validation():
    L = msa.lib()
    p = ctypes.c_void_p(16)
    d = base_desc(num_landmarks=3)
    assert L.msa_pool_landmarks(ctypes.byref(d), p, p, p, p, None) == 1
    d = base_desc(num_landmarks=0)
    assert L.msa_pool_landmarks(ctypes.byref(d), None, None, None, None, None) == 0


# ------------------------------------------------------------------ plans

SHAPES = [
    # (n, w, G) -- the workload shapes, then ragged and degenerate ones
    (2048, 256, 16), (32768, 4096, 512), (131072, 4096, 512),
    (64, 1, 0), (64, 64, 64), (192, 50, 3), (320, 1000, 5), (130, 7, 0), (1, 1, 0), (1, 1, 1),
    (100, 3, 10), (4096, 128, 4096), (777, 100, 7), (65, 65, 13),
]


@pytest.mark.parametrize("n,w,G", SHAPES + [(1048576, 4096, 512)])
@pytest.mark.parametrize("dtype", [msa.MSA_DTYPE_BF16, msa.MSA_DTYPE_F32])
def test_plan_rows_bitexact(n, w, G, dtype):
    d = base_desc(seq_len=n, window=w, num_landmarks=G, in_dtype=dtype, out_dtype=dtype)
    win_lo, lm = msa.msa_plan_rows(d)
    if n > 200000:
        rows = np.unique(np.concatenate([np.arange(0, 3 * w), np.random.default_rng(0).choice(n, 20000),
                                         np.arange(n - 2 * w, n)]))
    else:
        rows = np.arange(n)
    o_lo, o_lm = orc.row_plan(n, w, G, rows)
    np.testing.assert_array_equal(win_lo[rows], o_lo)
    np.testing.assert_array_equal(lm[rows], o_lm)


@pytest.mark.parametrize("n,w,G", SHAPES + [(1048576, 4096, 512)])
@pytest.mark.parametrize("dtype", [msa.MSA_DTYPE_BF16, msa.MSA_DTYPE_F32])
def test_plan_tiles_bitexact(n, w, G, dtype):
    d = base_desc(seq_len=n, window=w, num_landmarks=G, in_dtype=dtype, out_dtype=dtype)
    tiles, bm, bn = msa.msa_plan_tiles(d)
    T = -(-n // bm)
    if T > 300:
        rng = np.random.default_rng(1)
        qt = sorted(set(range(0, 40)) | set(range(T - 8, T)) | set(rng.choice(T, 60, replace=False).tolist()))
    else:
        qt = list(range(T))
    want = orc.tile_plan(n, w, G, bm, bn, q_tiles=qt)
    sel = np.isin(tiles[:, 0], qt)
    got = [tuple(int(x) for x in r[:3]) + (bool(r[3]),) for r in tiles[sel]]
    assert got == want
    # every query tile appears (each row sees at least itself)
    assert set(tiles[:, 0].tolist()) == set(range(T))


def test_plan_tile_counts_workloads():
    # Visible-tile totals per head for the 128K and 1M workloads: the
    # window part is w/bn + bm/bn (+1 for a straddling start) tiles per
    # query tile once past the ramp.
    for cfg in (wl.GQA_128K, wl.GQA_1M):
        d = base_desc(seq_len=cfg.seq_len, window=cfg.window, num_landmarks=cfg.num_landmarks)
        tiles, bm, bn = msa.msa_plan_tiles(d)
        win = tiles[tiles[:, 1] == 1]
        per_t = np.bincount(win[:, 0])
        T = cfg.seq_len // bm
        assert per_t[cfg.window // bm:].max() == cfg.window // bn + bm // bn
        assert per_t.sum() <= T * (cfg.window // bn + bm // bn)


@pytest.mark.parametrize("ctx,w,G,S", [(524288, 4096, 512, 16), (512, 64, 8, 4), (100, 1000, 0, 3),
                                        (64, 8, 8, 40), (4096, 300, 16, 7), (1, 1, 1, 2)])
def test_plan_decode_bitexact(ctx, w, G, S):
    d = dec_desc(ctx_len=ctx, window=w, num_landmarks=G, num_splits=S)
    bounds, lm, ent = msa.msa_plan_decode(d)
    kinds, idx = orc.visible_list(ctx - 1, ctx, w, G)
    assert ent == len(idx)
    assert lm == int((kinds == 0).sum())
    np.testing.assert_array_equal(bounds, orc.chunk_bounds(len(idx), S))


# ---------------------------------------------------------- incremental decode

@pytest.mark.parametrize("kw,status", [
    (dict(num_splits=0), 1), (dict(window=0), 1), (dict(num_landmarks=7), 1), (dict(ctx_len=0), 1),
    (dict(heads_q=40, heads_kv=2), 2), (dict(head_dim=96), 2),
    (dict(in_dtype=msa.MSA_DTYPE_F32), 2), (dict(ctx_len=1 << 23), 2),
])
def test_decode_varlen_validation(kw, status):
    d = dec_desc(**kw)
    p = ctypes.c_void_p(16)
    assert msa.lib().msa_decode_fwd_varlen(ctypes.byref(d), p, p, p, p, p, p, p, 1 << 30, p, None, None) == status


def test_decode_varlen_pointer_checks():
    d = dec_desc()
    p = ctypes.c_void_p(16)
    f = msa.lib().msa_decode_fwd_varlen
    assert f(ctypes.byref(d), None, p, p, p, p, p, p, 1 << 30, p, None, None) == 1
    assert b"ctx_lens" in msa.lib().msa_last_error()
    assert f(ctypes.byref(d), ctypes.c_void_p(18), p, p, p, p, p, p, 1 << 30, p, None, None) == 1
    assert f(ctypes.byref(d), ctypes.c_void_p(20), p, p, p, p, p, p, 16, p, None, None) == 3
    d0 = dec_desc(batch=0)
    assert f(ctypes.byref(d0), None, None, None, None, None, None, None, 0, None, None, None) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(ctx_len=0), 1), (dict(heads_kv=0), 1), (dict(num_landmarks=7), 1), (dict(head_dim=96), 2),
    (dict(in_dtype=msa.MSA_DTYPE_F32), 2), (dict(ctx_len=1 << 23), 2),
])
def test_append_validation(kw, status):
    d = dec_desc(**kw)
    p = ctypes.c_void_p(16)
    assert msa.lib().msa_append_kv(ctypes.byref(d), p, p, p, p, p, p, p, None) == status


def test_append_pointer_checks():
    d = dec_desc()
    p = ctypes.c_void_p(16)
    f = msa.lib().msa_append_kv
    assert f(ctypes.byref(d), None, p, p, p, p, p, p, None) == 1
    assert f(ctypes.byref(d), ctypes.c_void_p(18), p, p, p, p, p, p, None) == 1
    assert f(ctypes.byref(d), p, ctypes.c_void_p(24), p, p, p, p, p, None) == 1
    assert f(ctypes.byref(d), p, p, p, p, p, None, p, None) == 1
    assert b"Kbar" in msa.lib().msa_last_error()
    d0 = dec_desc(batch=0)
    assert f(ctypes.byref(d0), None, None, None, None, None, None, None, None) == 0


@pytest.mark.parametrize("C,w,G,S", [(524288, 4096, 512, 16), (512, 64, 8, 4), (100, 1000, 0, 3),
                                      (64, 8, 8, 40), (4096, 300, 16, 7)])
def test_plan_decode_varlen_bitexact(C, w, G, S):
    d = dec_desc(ctx_len=C, window=w, num_landmarks=G, num_splits=S)
    L = C // G if G else 1
    rng = np.random.default_rng(C + w)
    lens = sorted({0, 1, 2, C, C - 1, w, w + 1} | set(rng.integers(0, C + 1, 25).tolist()))
    for n in lens:
        if n > C:
            continue
        bounds, lm, ent = msa.msa_plan_decode_varlen(d, n)
        kinds, idx = orc.visible_list_fixed(n - 1, w, L, G) if n else (np.zeros(0), np.zeros(0))
        assert ent == len(idx), n
        assert lm == int((kinds == 0).sum()), n
        np.testing.assert_array_equal(bounds, orc.chunk_bounds(len(idx), S))
    with pytest.raises(msa.MsaError):
        msa.msa_plan_decode_varlen(d, C + 1)
    with pytest.raises(msa.MsaError):
        msa.msa_plan_decode_varlen(d, -1)
    # the full length is the static plan
    np.testing.assert_array_equal(msa.msa_plan_decode_varlen(d, C)[0], msa.msa_plan_decode(d)[0])


# ---------------------------------------------------------- backward

def call_bwd(desc, ws_bytes=1 << 40, ptr=16, **none):
    p = ctypes.c_void_p(ptr)
    args = {k: p for k in ("Q", "K", "V", "Kb", "Vb", "O", "LSE", "dO", "ws", "dQ", "dK", "dV")}
    for k in none:
        args[k] = None
    return msa.lib().msa_attn_bwd(ctypes.byref(desc), args["Q"], args["K"], args["V"], args["Kb"], args["Vb"],
                                  args["O"], args["LSE"], args["dO"], args["ws"], ws_bytes, args["dQ"],
                                  args["dK"], args["dV"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(window=0), 1), (dict(num_landmarks=3), 1), (dict(heads_q=3), 1), (dict(head_dim=96), 2),
    (dict(in_dtype=msa.MSA_DTYPE_F32, out_dtype=msa.MSA_DTYPE_F32), 2), (dict(seq_len=1 << 23), 2),
    (dict(scale=0.0), 1), (dict(out_dtype=7), 1),
])
def test_bwd_validation(kw, status):
    assert call_bwd(base_desc(**kw)) == status


def test_bwd_pointer_and_workspace_checks():
    d = base_desc()
    for name in ("Q", "K", "V", "O", "LSE", "dO", "ws", "dQ", "dK", "dV", "Kb", "Vb"):
        assert call_bwd(d, **{name: 1}) == 1, name
    assert call_bwd(d, ptr=24) == 1
    need = msa.msa_attn_bwd_workspace_size(d)
    assert call_bwd(d, ws_bytes=need - 1) == 3
    # without landmarks Kbar/Vbar may be NULL: the call gets past them to the
    # workspace check (no call here reaches a launch)
    assert call_bwd(base_desc(num_landmarks=0), Kb=1, Vb=1, ws_bytes=0) == 3
    d0 = base_desc(batch=0)
    assert call_bwd(d0, ptr=0) == 0


def test_bwd_workspace_size_formula():
    # (lse2, D) per padded row, plus two [B*Hkv][G][2][d] float32 arrays of
    # landmark gradients (per-segment partials and their sum)
    for n, G in ((256, 4), (131072, 512), (1000, 0), (1048576, 512)):
        d = base_desc(seq_len=n, num_landmarks=G, heads_q=64, heads_kv=8)
        got = msa.msa_attn_bwd_workspace_size(d)
        n_pad = -(-n // 128) * 128
        seg = max(1024, -(-n // 128))
        seg = -(-seg // 32) * 32
        nseg = -(-n // seg) if G else 0
        up = lambda x: -(-x // 256) * 256
        lm = 8 * G * 2 * 128 * 4
        assert got == up(64 * n_pad * 8) + up(nseg * lm) + up(lm)


# ---------------------------------------------------------- block-sparse lists

def call_list(desc, counts=16, idx=16, max_blocks=4, causal=1, ptr=16, lse=20):
    # LSE defaults to a misaligned address, so that a call passing every
    # other check still fails validation and nothing is launched
    p = ctypes.c_void_p(ptr)
    c = None if counts is None else ctypes.c_void_p(counts)
    i = None if idx is None else ctypes.c_void_p(idx)
    return msa.lib().msa_attn_fwd_blocksparse(ctypes.byref(desc), c, i, max_blocks, causal, p, p, p, p,
                                              ctypes.c_void_p(lse), None)


@pytest.mark.parametrize("kw,status", [
    (dict(heads_q=3), 1), (dict(head_dim=96), 2), (dict(scale=0.0), 1),
    (dict(in_dtype=msa.MSA_DTYPE_F32, out_dtype=msa.MSA_DTYPE_F32), 2), (dict(seq_len=1 << 23), 2),
])
def test_blocksparse_validation(kw, status):
    assert call_list(base_desc(**kw)) == status


def test_blocksparse_ignores_window_and_landmarks():
    # window and num_landmarks are not read: values that prefill rejects pass validation
    d = base_desc(window=0, num_landmarks=7)
    assert call_list(d, counts=None) == 1          # fails later, on the NULL counts
    assert b"block_counts" in msa.lib().msa_last_error()


def test_blocksparse_argument_checks():
    d = base_desc()
    assert call_list(d, max_blocks=-1) == 1
    assert call_list(d, causal=2) == 1
    assert call_list(d, counts=18) == 1
    assert call_list(d, idx=None) == 1
    assert call_list(d, idx=None, max_blocks=0) == 1   # no index array needed for empty lists:
    assert b"LSE" in msa.lib().msa_last_error()         # it fails on the LSE check that comes after
    assert call_list(d, ptr=24) == 1
    assert call_list(base_desc(batch=0), counts=None, idx=None, ptr=0) == 0


# ---------------------------------------------------------- paged caches

def call_paged(desc, page=64, num_pages=8, table=16, lens=16, lse=20):
    # LSE misaligned by default: a call passing every other check still fails
    # validation, so nothing is launched
    p = ctypes.c_void_p(16)
    t = None if table is None else ctypes.c_void_p(table)
    ln = None if lens is None else ctypes.c_void_p(lens)
    return msa.lib().msa_decode_fwd_paged(ctypes.byref(desc), page, num_pages, t, ln, p, p, p, p, p, p, 1 << 30,
                                          p, ctypes.c_void_p(lse), None)


@pytest.mark.parametrize("kw,status", [
    (dict(page=16), 1), (dict(page=48), 1), (dict(page=1024), 1), (dict(num_pages=0), 1),
    (dict(table=None), 1), (dict(table=18), 1), (dict(lens=None), 1), (dict(lens=22), 1),
])
def test_paged_decode_validation(kw, status):
    d = dec_desc(ctx_len=512, num_landmarks=8)   # capacity 512: page 1024 does not divide it
    assert call_paged(d, **kw) == status


def test_paged_decode_passes_to_the_last_check():
    d = dec_desc(ctx_len=512, num_landmarks=8)
    assert call_paged(d) == 1 and b"LSE" in msa.lib().msa_last_error()
    # pools are addressed in 64 bits: a capacity over 2 GiB per head is accepted
    big = dec_desc(ctx_len=1 << 23, num_landmarks=8)
    assert call_paged(big, page=1 << 16) == 1 and b"LSE" in msa.lib().msa_last_error()
    # a contiguous decode of that capacity is refused
    p = ctypes.c_void_p(16)
    assert msa.lib().msa_decode_fwd(ctypes.byref(big), p, p, p, p, p, p, 1 << 30, p, None, None) == 2


def test_paged_append_validation():
    d = dec_desc(ctx_len=512, num_landmarks=8)
    p = ctypes.c_void_p(16)
    f = msa.lib().msa_append_kv_paged
    assert f(ctypes.byref(d), 48, 8, p, p, p, p, p, p, p, p, None) == 1
    assert f(ctypes.byref(d), 64, 0, p, p, p, p, p, p, p, p, None) == 1
    assert f(ctypes.byref(d), 64, 8, None, p, p, p, p, p, p, p, None) == 1
    assert f(ctypes.byref(d), 64, 8, p, None, p, p, p, p, p, p, None) == 1
    assert f(ctypes.byref(d), 64, 8, p, p, p, p, p, p, None, p, None) == 1   # Kbar needed with G > 0
    assert f(ctypes.byref(dec_desc(in_dtype=msa.MSA_DTYPE_F32)), 64, 8, p, p, p, p, p, p, p, p, None) == 2
    assert f(ctypes.byref(dec_desc(batch=0)), 48, 0, None, None, None, None, None, None, None, None, None) == 0


def test_noalloc_decode_rejects_partials_beyond_its_array():
    # 64 sequences x 64 query heads x 16 chunks x 129 floats = 33,816,576 B of
    # partials under the split schedule: more than the library's 32 MiB
    d = dec_desc(batch=64, heads_q=64, heads_kv=8, ctx_len=4096, window=1024, num_landmarks=8, num_splits=16,
                 schedule=msa.MSA_DECODE_SPLIT)
    p = ctypes.c_void_p(16)
    L = msa.lib()
    assert L.msa_decode_fwd_noalloc(ctypes.byref(d), p, p, p, p, p, p, None, None) == 3  # MSA_ERR_WORKSPACE
    assert b"33816576 bytes of partials" in L.msa_last_error()
    assert L.msa_decode_fwd_noalloc(ctypes.byref(d), None, p, p, p, p, p, None, None) == 1


def test_reference_library_loads_and_rejects_bad_arguments():
    """bench.py's measured references live in libmsa_ref.so, outside the
    library's interface: it loads, exports msa_ref_mfma, and refuses a bad
    mode or count before touching the GPU."""
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "long_context_sparse_msa_amd", "libmsa_ref.so")
    if not os.path.exists(path):
        pytest.skip("libmsa_ref.so not built")
    ref = ctypes.CDLL(path)
    f = ref.msa_ref_mfma
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                  ctypes.POINTER(ctypes.c_double)]
    ms, fl = ctypes.c_double(), ctypes.c_double()
    for mode, iters, reps in ((2, 10, 1), (-1, 10, 1), (0, 0, 1), (1, 10, 0)):
        assert f(mode, iters, reps, ctypes.byref(ms), ctypes.byref(fl)) != 0
    assert f(0, 10, 1, None, ctypes.byref(fl)) != 0


def _random_shapes(count, seed):
    """Seeded (n, w, G) with G = 0 or a divisor of n (n = G * L), windows from
    1 to beyond n, and n from 1 to a few thousand."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        L = int(rng.integers(1, 300))
        G = int(rng.integers(0, 24))
        n = G * L if G > 0 else int(rng.integers(1, 5000))
        if n < 1 or n > 6000:
            continue
        w = int(rng.choice([1, 2, 63, 64, 65, int(rng.integers(1, n + 1)), n, 2 * n + 3]))
        out.append((n, max(1, w), G))
    return out


@pytest.mark.parametrize("n,w,G", _random_shapes(60, 11))
def test_plan_rows_and_tiles_bitexact_random(n, w, G):
    """Seeded random shapes (ragged n, landmark blocks of any length, windows
    shorter and longer than n): the library's row and tile plans equal the
    oracle's mask-derived ones exactly."""
    d = base_desc(seq_len=n, window=w, num_landmarks=G)
    win_lo, lm = msa.msa_plan_rows(d)
    rows = np.arange(n)
    o_lo, o_lm = orc.row_plan(n, w, G, rows)
    np.testing.assert_array_equal(win_lo, o_lo)
    np.testing.assert_array_equal(lm, o_lm)
    tiles, bm, bn = msa.msa_plan_tiles(d)
    T = -(-n // bm)
    want = orc.tile_plan(n, w, G, bm, bn, q_tiles=list(range(T)))
    got = [tuple(int(x) for x in r[:3]) + (bool(r[3]),) for r in tiles]
    assert got == want


@pytest.mark.parametrize("ctx,w,G,S", [(s[0], s[1], s[2], int(k)) for s, k in
                                       zip(_random_shapes(40, 12), np.random.default_rng(13).integers(1, 40, 40))])
def test_plan_decode_bitexact_random(ctx, w, G, S):
    d = dec_desc(ctx_len=ctx, window=w, num_landmarks=G, num_splits=S)
    bounds, lm, ent = msa.msa_plan_decode(d)
    kinds, idx = orc.visible_list(ctx - 1, ctx, w, G)
    assert ent == len(idx)
    assert lm == int((kinds == 0).sum())
    np.testing.assert_array_equal(bounds, orc.chunk_bounds(len(idx), S))
