"""Pins of the oracle's block-sparse-list attention against facts fixed
outside it: lists that spell out the window pattern give the pinned window
attention, full causal lists give torch's causal SDPA, a pure-Python loop
on tiny inputs, listing a block twice doubles its weight, and rows that see
nothing."""
import math

import numpy as np
import pytest
import torch

from oracle import msa_oracle as orc

SC = 0.3


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def lists_from(fn, B, H, T, maxb):
    counts = np.zeros((B, H, T), np.int32)
    idx = np.full((B, H, T, maxb), -1, np.int32)
    for b in range(B):
        for h in range(H):
            for t in range(T):
                blocks = fn(b, h, t)
                counts[b, h, t] = len(blocks)
                idx[b, h, t, :len(blocks)] = blocks
    return counts, idx


def test_full_causal_lists_are_causal_sdpa():
    n, bq, bk = 96, 32, 16
    Q, K, V = rnd((1, 2, n, 8), 1), rnd((1, 2, n, 8), 2), rnd((1, 2, n, 8), 3)
    T, nkb = n // bq, n // bk
    counts, idx = lists_from(lambda b, h, t: list(range(nkb)), 1, 2, T, nkb)
    O, L = orc.attn_blocksparse(Q, K, V, counts, idx, bq, bk, True, SC)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x) for x in (Q, K, V)), is_causal=True, scale=SC).numpy()
    np.testing.assert_allclose(O, ref, atol=1e-12)


@pytest.mark.parametrize("w_blocks", [1, 2, 3])
def test_block_window_lists_equal_window_attention_on_aligned_rows(w_blocks):
    # causal lists of the w_blocks key blocks ending at the query block: for
    # the last row of each query block (bq == bk) the visible keys are
    # exactly the window of w = w_blocks*bk keys, so it matches the pinned
    # window attention without landmarks there
    n, bs = 128, 16
    Q, K, V = rnd((1, 1, n, 8), 4), rnd((1, 1, n, 8), 5), rnd((1, 1, n, 8), 6)
    T = n // bs
    counts, idx = lists_from(lambda b, h, t: list(range(max(0, t - w_blocks + 1), t + 1)), 1, 1, T, w_blocks)
    O, L = orc.attn_blocksparse(Q, K, V, counts, idx, bs, bs, True, SC)
    Ow, Lw = orc.attn_dense(Q, K, V, w_blocks * bs, 0, SC)
    last = np.arange(bs - 1, n, bs)
    np.testing.assert_allclose(O[:, :, last], Ow[:, :, last], atol=1e-12)
    np.testing.assert_allclose(L[:, :, last], Lw[:, :, last], atol=1e-12)


def brute(Q, K, V, counts, idx, bq, bk, causal, scale):
    B, H, n, d = Q.shape
    O = np.zeros((B, H, n, d))
    L = np.full((B, H, n), -np.inf)
    nkb = -(-n // bk)
    for b in range(B):
        for h in range(H):
            for i in range(n):
                t = i // bq
                ents = []
                for c in range(counts[b, h, t]):
                    kb = idx[b, h, t, c]
                    if not 0 <= kb < nkb:
                        continue
                    for j in range(kb * bk, min(n, kb * bk + bk)):
                        if causal and j > i:
                            continue
                        ents.append((scale * sum(Q[b, h, i, e] * K[b, h, j, e] for e in range(d)), j))
                if not ents:
                    continue
                m = max(s for s, _ in ents)
                l = sum(math.exp(s - m) for s, _ in ents)
                for e in range(d):
                    O[b, h, i, e] = sum(math.exp(s - m) * V[b, h, j, e] for s, j in ents) / l
                L[b, h, i] = m + math.log(l)
    return O, L


@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_random_lists(causal):
    n, bq, bk = 20, 8, 4
    Q, K, V = rnd((2, 2, n, 3), 7), rnd((2, 2, n, 3), 8), rnd((2, 2, n, 3), 9)
    rng = np.random.default_rng(10)
    T, nkb = -(-n // bq), -(-n // bk)
    counts, idx = lists_from(lambda b, h, t: list(rng.integers(-1, nkb + 1, size=rng.integers(0, 5))), 2, 2, T, 4)
    O, L = orc.attn_blocksparse(Q, K, V, counts, idx, bq, bk, causal, SC)
    Ob, Lb = brute(Q, K, V, counts, idx, bq, bk, causal, SC)
    np.testing.assert_allclose(O, Ob, atol=1e-12)
    np.testing.assert_allclose(L, Lb, atol=1e-12)


def test_block_listed_twice_counts_twice():
    # every score of a block listed twice enters the softmax twice:
    # equivalent to adding ln 2 to those scores
    n, bs = 32, 8
    Q, K, V = rnd((1, 1, n, 4), 11), rnd((1, 1, n, 4), 12), rnd((1, 1, n, 4), 13)
    counts, idx = lists_from(lambda b, h, t: [0, 1, 1], 1, 1, n // bs, 3)
    O, L = orc.attn_blocksparse(Q, K, V, counts, idx, bs, bs, False, SC)
    S = SC * Q[0, 0] @ K[0, 0, :16].T
    S[:, 8:] += np.log(2.0)
    P = np.exp(S - S.max(1, keepdims=True))
    np.testing.assert_allclose(O[0, 0], (P / P.sum(1, keepdims=True)) @ V[0, 0, :16], atol=1e-12)


def test_rows_that_see_nothing():
    n, bs = 32, 8
    Q, K, V = rnd((1, 1, n, 4), 14), rnd((1, 1, n, 4), 15), rnd((1, 1, n, 4), 16)
    # query block 0 lists nothing; block 1 lists only a later block (causal hides it)
    counts, idx = lists_from(lambda b, h, t: [] if t == 0 else ([3] if t == 1 else [t]), 1, 1, n // bs, 1)
    O, L = orc.attn_blocksparse(Q, K, V, counts, idx, bs, bs, True, SC)
    assert (O[0, 0, :16] == 0).all() and np.isneginf(L[0, 0, :16]).all()
    assert np.isfinite(L[0, 0, 16:]).all()


@pytest.mark.parametrize("causal", [False, True])
def test_rows_version_equals_dense(causal):
    n, bq, bk = 200, 32, 16
    Q, K, V = rnd((2, 4, n, 8), 20), rnd((2, 2, n, 8), 21), rnd((2, 2, n, 8), 22)
    rng = np.random.default_rng(23)
    T, nkb = -(-n // bq), -(-n // bk)
    counts, idx = lists_from(lambda b, h, t: list(rng.integers(-2, nkb + 2, size=rng.integers(0, 9))), 2, 4, T, 8)
    O, L = orc.attn_blocksparse(Q, K, V, counts, idx, bq, bk, causal, SC)
    rows = {h: np.sort(np.random.default_rng(h).choice(n, 30, replace=False)) for h in (0, 3)}
    for h, (r, o, l) in orc.attn_blocksparse_rows(Q, K, V, counts, idx, bq, bk, causal, SC, rows).items():
        np.testing.assert_allclose(o, O[:, h, r], atol=1e-12)
        np.testing.assert_allclose(l, L[:, h, r], atol=1e-12)
