"""Pins of the oracle's incremental decode (sequences of different lengths
in one cache, landmark blocks of a fixed length L, one token appended per
step) against facts fixed outside it: the already pinned prefill of a padded
sequence, textbook causal attention, closed-form landmark values and
sequence independence."""
import numpy as np
import pytest
import torch

from oracle import msa_oracle as orc

SC = 0.3


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def garbage_cache(B, Hkv, C, d, lens, seed):
    """Random cache whose rows at or past each sequence's length are large,
    so that reading them would change the result visibly."""
    K, V = rnd((B, Hkv, C, d), seed), rnd((B, Hkv, C, d), seed + 1)
    for b, n in enumerate(lens):
        K[b, :, n:] *= 40.0
        V[b, :, n:] = 1e3
    return K, V


# ------------------------------------------------------------ decode_varlen

VARLEN_CASES = [(n, w, L) for n in (1, 5, 16, 17, 31, 48, 63) for w in (1, 3, 8, 70) for L in (1, 4, 8)]


@pytest.mark.parametrize("n,w,L", VARLEN_CASES)
def test_varlen_equals_prefill_row_of_padded_sequence(n, w, L):
    # A sequence of n tokens in a cache of capacity C = G_cap*L: its decode
    # is row n-1 of the prefill over the first m = ceil(n/L)*L rows with
    # m/L landmarks (row n-1 never sees the incomplete block, nor any row
    # past n-1, so what those rows hold does not matter).
    G_cap = 64 // L
    C = G_cap * L
    m = -(-n // L) * L
    d, Hq, Hkv = 8, 4, 2
    Kc, Vc = garbage_cache(1, Hkv, C, d, [n], 100 + n)
    Q = rnd((1, Hq, m, d), 200 + w)
    O, LSE = orc.attn_dense(Q, Kc[:, :, :m], Vc[:, :, :m], w, m // L, SC)
    Od, Ld = orc.decode_varlen(Q[:, :, n - 1], Kc, Vc, [n], w, L, G_cap, SC)
    np.testing.assert_allclose(Od, O[:, :, n - 1], atol=1e-12)
    np.testing.assert_allclose(Ld, LSE[:, :, n - 1], atol=1e-12)


@pytest.mark.parametrize("n", [1, 2, 9, 40])
def test_varlen_window_covers_everything_is_textbook_causal(n):
    # w >= n: no landmark is visible and the last row is causal attention
    C, L, d = 64, 8, 16
    Kc, Vc = garbage_cache(1, 2, C, d, [n], 300 + n)
    q = rnd((1, 2, d), 301)
    Od, Ld = orc.decode_varlen(q, Kc, Vc, [n], n + 5, L, C // L, SC)
    Qm = torch.zeros((1, 2, n, d), dtype=torch.float64)
    Qm[:, :, -1] = torch.from_numpy(q)
    ref = torch.nn.functional.scaled_dot_product_attention(
        Qm, torch.from_numpy(Kc[:, :, :n]), torch.from_numpy(Vc[:, :, :n]), is_causal=True, scale=SC)
    np.testing.assert_allclose(Od, ref[:, :, -1].numpy(), atol=1e-12)
    s = SC * np.einsum("hd,hjd->hj", q[0], Kc[0, :, :n])
    np.testing.assert_allclose(Ld[0], np.log(np.exp(s).sum(-1)), atol=1e-12)


def test_varlen_sequences_are_independent():
    lens = [57, 8, 64, 33]
    C, L, w, d = 64, 8, 12, 8
    Kc, Vc = garbage_cache(4, 2, C, d, lens, 400)
    q = rnd((4, 4, d), 401)
    O, LSE = orc.decode_varlen(q, Kc, Vc, lens, w, L, C // L, SC)
    for b, n in enumerate(lens):
        Ob, Lb = orc.decode_varlen(q[b:b + 1], Kc[b:b + 1], Vc[b:b + 1], [n], w, L, C // L, SC)
        np.testing.assert_allclose(O[b], Ob[0], atol=1e-13)
        np.testing.assert_allclose(LSE[b], Lb[0], atol=1e-13)


def test_varlen_full_lengths_equal_static_decode():
    C, L, w = 128, 16, 20
    Kc, Vc = rnd((2, 2, C, 8), 410), rnd((2, 2, C, 8), 411)
    q = rnd((2, 4, 8), 412)
    O, LSE = orc.decode_varlen(q, Kc, Vc, [C, C], w, L, C // L, SC)
    Os, Ls = orc.decode(q, Kc, Vc, w, C // L, SC)
    np.testing.assert_allclose(O, Os, atol=1e-13)
    np.testing.assert_allclose(LSE, Ls, atol=1e-13)


@pytest.mark.parametrize("S", [1, 3, 7, 40])
def test_varlen_split_merge_equals_unsplit(S):
    lens = [3, 64, 29, 50]
    C, L, w = 64, 4, 9
    Kc, Vc = garbage_cache(4, 1, C, 8, lens, 420)
    q = rnd((4, 2, 8), 421)
    O1, L1 = orc.decode_varlen(q, Kc, Vc, lens, w, L, C // L, SC)
    o, lse = orc.decode_varlen_partials(q, Kc, Vc, lens, w, L, C // L, S, SC)
    O, LS = orc.merge(o, lse)
    np.testing.assert_allclose(O, O1, atol=1e-13)
    np.testing.assert_allclose(LS, L1, atol=1e-13)
    for b, n in enumerate(lens):
        E = len(orc.visible_list_fixed(n - 1, w, L, C // L)[1])
        s = -(-E // S)
        for c in range(S):
            assert np.isfinite(lse[c, b]).all() == (c * s < E)


def test_varlen_empty_sequence():
    Kc, Vc = rnd((2, 1, 32, 8), 430), rnd((2, 1, 32, 8), 431)
    O, LSE = orc.decode_varlen(rnd((2, 2, 8), 432), Kc, Vc, [0, 32], 4, 4, 8, SC)
    assert (O[0] == 0).all() and np.isneginf(LSE[0]).all()
    assert np.isfinite(LSE[1]).all()


def test_visible_list_fixed_example():
    # i = 99, w = 30, L = 10: blocks whose last position 10b+9 <= 69 -> b <= 6
    kinds, idx = orc.visible_list_fixed(99, 30, 10, 20)
    assert list(kinds) == [0] * 7 + [1] * 30
    assert list(idx) == list(range(7)) + list(range(70, 100))
    # i = 104 (a length of 105, not a multiple of L): the same blocks, since
    # block 7 ends at 79 > 74
    kinds, idx = orc.visible_list_fixed(104, 30, 10, 20)
    assert list(idx[kinds == 0]) == list(range(7))
    assert list(idx[kinds == 1]) == list(range(75, 105))


# ---------------------------------------------------------------- append

def test_append_builds_closed_form_landmarks():
    # row p holds p * c: block b's mean is c * (b*L + (L-1)/2)
    B, Hkv, C, d, L = 2, 2, 48, 4, 6
    c = np.array([1.0, -0.5, 0.25, 2.0])
    Kc, Vc = np.zeros((B, Hkv, C, d)), np.zeros((B, Hkv, C, d))
    Kb, Vb = np.zeros((B, Hkv, C // L, d)), np.zeros((B, Hkv, C // L, d))
    start = [0, L]  # sequence 1 never writes block 0, which stays zero
    for t in range(C):
        pos = np.array([t + start[0], t + start[1]])
        kn = np.stack([np.broadcast_to(p * c, (Hkv, d)) for p in pos])
        orc.append_tokens(Kc, Vc, Kb, Vb, pos, kn, -kn, L)
        for b in range(B):
            done = min(C, t + start[b] + 1) // L
            for blk in range(C // L):
                filled = blk < done and not (b == 1 and blk == 0)
                want = c * (blk * L + (L - 1) / 2) if filled else np.zeros(d)
                np.testing.assert_allclose(Kb[b, :, blk], np.broadcast_to(want, (Hkv, d)), atol=1e-12)
                np.testing.assert_allclose(Vb[b, :, blk], -np.broadcast_to(want, (Hkv, d)), atol=1e-12)


def test_append_positions_out_of_range_change_nothing():
    Kc, Vc = rnd((3, 2, 16, 4), 440), rnd((3, 2, 16, 4), 441)
    Kb, Vb = rnd((3, 2, 4, 4), 442), rnd((3, 2, 4, 4), 443)
    before = [x.copy() for x in (Kc, Vc, Kb, Vb)]
    kn = rnd((3, 2, 4), 444)
    orc.append_tokens(Kc, Vc, Kb, Vb, [-1, 16, 3], kn, kn, 4)
    for x, y in zip((Kc, Vc), before[:2]):
        np.testing.assert_array_equal(x[:2], y[:2])
        np.testing.assert_array_equal(x[2, :, :3], y[2, :, :3])
        np.testing.assert_array_equal(x[2, :, 4:], y[2, :, 4:])
    np.testing.assert_array_equal(Kc[2, :, 3], kn[2])
    np.testing.assert_array_equal(Kb[:2], before[2][:2])
    # position 3 completes block 0 of sequence 2 (L = 4)
    np.testing.assert_allclose(Kb[2, :, 0], Kc[2, :, 0:4].mean(axis=1), atol=1e-15)
    np.testing.assert_array_equal(Kb[2, :, 1:], before[2][2, :, 1:])


def test_append_then_decode_equals_decode_of_the_whole_prefix():
    # tokens appended one by one, decoding after each step, equal the decode
    # of a cache written at once with its landmarks pooled
    B, Hkv, Hq, C, d, L, w = 2, 1, 2, 40, 8, 5, 7
    ks, vs = rnd((C, B, Hkv, d), 450), rnd((C, B, Hkv, d), 451)
    qs = rnd((C, B, Hq, d), 452)
    Kc, Vc = np.zeros((B, Hkv, C, d)), np.zeros((B, Hkv, C, d))
    Kb, Vb = np.zeros((B, Hkv, C // L, d)), np.zeros((B, Hkv, C // L, d))
    full_K, full_V = np.moveaxis(ks, 0, 2), np.moveaxis(vs, 0, 2)
    for t in range(C):
        orc.append_tokens(Kc, Vc, Kb, Vb, [t, t], ks[t], vs[t], L)
        O, LSE = orc.decode_varlen(qs[t], Kc, Vc, [t + 1, t + 1], w, L, C // L, SC, Kbar=Kb, Vbar=Vb)
        m = -(-(t + 1) // L) * L
        Qp = np.zeros((B, Hq, m, d))
        Qp[:, :, t] = qs[t]
        Kp, Vp = full_K[:, :, :m].copy(), full_V[:, :, :m].copy()
        Op, Lp = orc.attn_dense(Qp, Kp, Vp, w, m // L, SC)
        np.testing.assert_allclose(O, Op[:, :, t], atol=1e-12)
        np.testing.assert_allclose(LSE, Lp[:, :, t], atol=1e-12)


# ---------------------------------------------------------------- paging

def test_gather_pages_inverts_a_scatter():
    rng = np.random.default_rng(460)
    B, Hkv, P, page, d = 3, 2, 5, 4, 3
    X = rng.standard_normal((B, Hkv, P * page, d))
    perm = rng.permutation(B * P + 4)[:B * P].reshape(B, P)   # 4 pool pages stay unused
    pool = rng.standard_normal((B * P + 4, Hkv, page, d))
    for b in range(B):
        for lp in range(P):
            pool[perm[b, lp]] = X[b, :, lp * page:(lp + 1) * page]
    np.testing.assert_array_equal(orc.gather_pages(pool, perm, page), X)
    bad = perm.copy()
    bad[1, 2] = -1
    g = orc.gather_pages(pool, bad, page)
    assert (g[1, :, 8:12] == 0).all()
