"""Pins of the fp64 oracle against facts fixed outside it: brute force on
tiny inputs, reductions to textbook attention, closed forms, the hand-derived
worked example and the figures printed on the pages."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import msa_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- brute force

def brute_force(Q, K, V, w, G, scale):
    """Triple loop in plain Python floats with math.exp."""
    B, Hq, n, d = Q.shape
    Hkv = K.shape[1]
    grp = Hq // Hkv
    L = n // G if G else 0
    O = np.zeros((B, Hq, n, d))
    LSE = np.zeros((B, Hq, n))
    for b in range(B):
        for h in range(Hq):
            g = h // grp
            lmk = [[sum(float(K[b, g, blk * L + t, e]) for t in range(L)) / L for e in range(d)] for blk in range(G)]
            lmv = [[sum(float(V[b, g, blk * L + t, e]) for t in range(L)) / L for e in range(d)] for blk in range(G)]
            for i in range(n):
                ents = []
                for j in range(n):
                    if i - w < j <= i:
                        s = scale * sum(float(Q[b, h, i, e]) * float(K[b, g, j, e]) for e in range(d))
                        ents.append((s, [float(V[b, g, j, e]) for e in range(d)]))
                for blk in range(G):
                    if (blk + 1) * L - 1 <= i - w:
                        s = scale * sum(float(Q[b, h, i, e]) * lmk[blk][e] for e in range(d))
                        ents.append((s, lmv[blk]))
                m = max(s for s, _ in ents)
                l = sum(math.exp(s - m) for s, _ in ents)
                for e in range(d):
                    O[b, h, i, e] = sum(math.exp(s - m) * v[e] for s, v in ents) / l
                LSE[b, h, i] = m + math.log(l)
    return O, LSE


BRUTE_CASES = []
for n in (8, 12, 16, 24):
    for w in (1, 2, 3, 5, n, 2 * n):
        for G in [0] + [g for g in (1, 2, 3, 4, 6, 8, n) if n % g == 0]:
            BRUTE_CASES.append((n, w, G))


@pytest.mark.parametrize("n,w,G", BRUTE_CASES[::3] + [(16, 3, 4), (24, 5, 6), (24, 2, 24)])
def test_brute_force_mha(n, w, G):
    Q, K, V = rnd((1, 2, n, 4), 1), rnd((1, 2, n, 4), 2), rnd((1, 2, n, 4), 3)
    O, L = orc.attn_dense(Q, K, V, w, G, 0.7)
    Ob, Lb = brute_force(Q, K, V, w, G, 0.7)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, Lb, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n,w,G", [(16, 3, 4), (12, 4, 3), (16, 16, 16)])
def test_brute_force_gqa_batch(n, w, G):
    Q, K, V = rnd((2, 4, n, 3), 4), rnd((2, 2, n, 3), 5), rnd((2, 2, n, 3), 6)
    O, L = orc.attn_dense(Q, K, V, w, G, 0.5)
    Ob, Lb = brute_force(Q, K, V, w, G, 0.5)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, Lb, rtol=0, atol=1e-12)


# ---------------------------------------------------------- reductions

def numpy_causal(Q, K, V, scale):
    """Dense causal softmax attention, written independently of the oracle."""
    n = Q.shape[-2]
    S = scale * np.einsum("bhid,bhjd->bhij", Q, K)
    S = S + np.triu(np.full((n, n), -np.inf), 1)
    m = S.max(-1, keepdims=True)
    P = np.exp(S - m)
    l = P.sum(-1, keepdims=True)
    return np.einsum("bhij,bhjd->bhid", P / l, V), (m + np.log(l))[..., 0]


@pytest.mark.parametrize("n,w", [(64, 64), (64, 200), (96, 96)])
def test_full_window_no_landmarks_is_causal_sdpa(n, w):
    Q, K, V = rnd((1, 3, n, 16), 7), rnd((1, 3, n, 16), 8), rnd((1, 3, n, 16), 9)
    O, L = orc.attn_dense(Q, K, V, w, 0, 0.25)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q), torch.from_numpy(K), torch.from_numpy(V), is_causal=True, scale=0.25).numpy()
    np.testing.assert_allclose(O, ref, atol=1e-12)
    Oc, Lc = numpy_causal(Q, K, V, 0.25)
    np.testing.assert_allclose(O, Oc, atol=1e-12)
    np.testing.assert_allclose(L, Lc, atol=1e-12)


@pytest.mark.parametrize("w", [1, 2, 7, 33, 64])
def test_one_token_landmarks_give_causal_attention_for_any_window(w):
    # G = n makes each landmark a single key, visible iff b <= i - w, so the
    # window and the landmarks together cover exactly the keys j <= i.
    n = 64
    Q, K, V = rnd((1, 2, n, 8), 10), rnd((1, 2, n, 8), 11), rnd((1, 2, n, 8), 12)
    O, L = orc.attn_dense(Q, K, V, w, n, 0.3)
    Oc, Lc = numpy_causal(Q, K, V, 0.3)
    np.testing.assert_allclose(O, Oc, atol=1e-12)
    np.testing.assert_allclose(L, Lc, atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv():
    n, w, G = 64, 9, 8
    Q, K, V = rnd((2, 8, n, 8), 13), rnd((2, 2, n, 8), 14), rnd((2, 2, n, 8), 15)
    O, L = orc.attn_dense(Q, K, V, w, G, 0.4)
    Om, Lm = orc.attn_dense(Q, np.repeat(K, 4, axis=1), np.repeat(V, 4, axis=1), w, G, 0.4)
    np.testing.assert_allclose(O, Om, atol=1e-13)
    np.testing.assert_allclose(L, Lm, atol=1e-13)
    # and the mapping is by consecutive groups: moving one KV head changes
    # exactly the query heads of its group
    K2 = K.copy()
    K2[:, 1] *= 2.0
    O2, _ = orc.attn_dense(Q, K2, V, w, G, 0.4)
    changed = [h for h in range(8) if not np.allclose(O2[:, h], O[:, h])]
    assert changed == [4, 5, 6, 7]


# ---------------------------------------------------------- closed forms

def test_window_one_no_landmarks_is_identity():
    n = 40
    Q, K, V = rnd((1, 2, n, 8), 16), rnd((1, 2, n, 8), 17), rnd((1, 2, n, 8), 18)
    O, L = orc.attn_dense(Q, K, V, 1, 0, 0.6)
    np.testing.assert_allclose(O, V, atol=1e-14)
    np.testing.assert_allclose(L, 0.6 * np.einsum("bhid,bhid->bhi", Q, K), atol=1e-13)


def test_golden_uniform_worked_example():
    with open(os.path.join(GOLDEN, "uniform_n8_w2_G2.json")) as f:
        gold = json.load(f)
    n, d, w, G = gold["n"], gold["d"], gold["w"], gold["G"]
    V = np.array(gold["V"], dtype=np.float64)[None, None]
    K = np.zeros_like(V)
    Q = rnd((1, 1, n, d), 19)
    O, L = orc.attn_dense(Q, K, V, w, G, gold["scale"])
    want = np.array([[float(Fraction(x)) for x in r] for r in gold["O"]])
    np.testing.assert_allclose(O[0, 0], want, atol=1e-14)
    np.testing.assert_allclose(L[0, 0], np.log(gold["count"]), atol=1e-14)
    lm = np.array([[float(Fraction(x)) for x in r] for r in gold["landmark_V"]])
    np.testing.assert_allclose(orc.pool(V, G)[0, 0], lm, atol=1e-15)


@pytest.mark.parametrize("n,w,G", [(128, 16, 8), (128, 40, 4), (96, 7, 12)])
def test_zero_keys_average_the_visible_values(n, w, G):
    # With K = 0 every visible entry gets weight 1: O_i is the mean of the
    # visible value rows (window rows and landmark means), LSE_i = ln(count).
    # The visible sets are enumerated here straight from the stated rule.
    L = n // G
    V = rnd((1, 1, n, 5), 20)
    Q = rnd((1, 1, n, 5), 21)
    O, LSE = orc.attn_dense(Q, np.zeros_like(V), V, w, G, 1.0)
    for i in range(n):
        rows = [V[0, 0, j] for j in range(max(0, i - w + 1), i + 1)]
        rows += [V[0, 0, b * L:(b + 1) * L].mean(0) for b in range(G) if (b + 1) * L <= i - w + 1]
        np.testing.assert_allclose(O[0, 0, i], np.mean(rows, axis=0), atol=1e-13)
        assert abs(LSE[0, 0, i] - math.log(len(rows))) < 1e-13


def test_constant_values_pass_through():
    n, w, G = 64, 10, 8
    Q, K = rnd((1, 2, n, 6), 22), rnd((1, 2, n, 6), 23)
    c = rnd((6,), 24)
    V = np.broadcast_to(c, (1, 2, n, 6)).copy()
    O, _ = orc.attn_dense(Q, K, V, w, G, 0.5)
    np.testing.assert_allclose(O, np.broadcast_to(c, O.shape), atol=1e-13)


def test_key_shift_moves_lse_only():
    # Adding the same vector c to every key adds scale*q_i.c to every score
    # of row i (landmark means shift identically): O unchanged, LSE shifted.
    n, w, G = 64, 11, 4
    Q, K, V = rnd((1, 2, n, 6), 25), rnd((1, 2, n, 6), 26), rnd((1, 2, n, 6), 27)
    c = rnd((6,), 28)
    O, L = orc.attn_dense(Q, K, V, w, G, 0.5)
    O2, L2 = orc.attn_dense(Q, K + c, V, w, G, 0.5)
    np.testing.assert_allclose(O2, O, atol=1e-12)
    np.testing.assert_allclose(L2, L + 0.5 * np.einsum("bhid,d->bhi", Q, c), atol=1e-12)


def test_softmax_weights_for_powers_of_two():
    # d = 1, q = 1, k_j = j ln 2, scale 1: row i's window weights are 2^j,
    # so O_i = sum 2^j v_j / sum 2^j over the visible j and LSE_i = ln(sum 2^j).
    n, w = 10, 4
    Q = np.ones((1, 1, n, 1))
    K = (np.arange(n) * math.log(2.0)).reshape(1, 1, n, 1)
    V = rnd((1, 1, n, 1), 29)
    O, L = orc.attn_dense(Q, K, V, w, 0, 1.0)
    for i in range(n):
        js = range(max(0, i - w + 1), i + 1)
        den = sum(2.0 ** j for j in js)
        assert abs(O[0, 0, i, 0] - sum(2.0 ** j * V[0, 0, j, 0] for j in js) / den) < 1e-12
        assert abs(L[0, 0, i] - math.log(den)) < 1e-12


# ---------------------------------------------------------- pooling

def test_pool_constant_blocks_and_bruteforce():
    n, G, d = 64, 8, 3
    L = n // G
    X = np.repeat(np.round(rnd((2, 2, G, d), 30) * 16) / 16, L, axis=2)  # dyadic: sums exact
    np.testing.assert_array_equal(orc.pool(X, G), X[:, :, ::L])
    Y = rnd((2, 2, n, d), 31)
    P = orc.pool(Y, G)
    for b in range(G):
        for e in range(d):
            s = 0.0
            for t in range(L):
                s += Y[0, 1, b * L + t, e]
            assert abs(P[0, 1, b, e] - s / L) < 1e-14


def test_pool_rejects_non_divisor():
    with pytest.raises(ValueError):
        orc.pool(np.zeros((1, 1, 10, 2)), 3)


# ---------------------------------------------------------- split / decode

@pytest.mark.parametrize("ctx,w,G,S", [(256, 64, 16, 16), (256, 64, 16, 1), (256, 64, 16, 2),
                                        (64, 8, 8, 40), (200, 1000, 0, 3), (256, 32, 0, 16)])
def test_split_merge_equals_unsplit(ctx, w, G, S):
    q = rnd((2, 4, 8), 32)
    Kc, Vc = rnd((2, 2, ctx, 8), 33), rnd((2, 2, ctx, 8), 34)
    O1, L1 = orc.decode(q, Kc, Vc, w, G, 0.35)
    o, lse = orc.decode_partials(q, Kc, Vc, w, G, S, 0.35)
    O, L = orc.merge(o, lse)
    np.testing.assert_allclose(O, O1, atol=1e-13)
    np.testing.assert_allclose(L, L1, atol=1e-13)
    # chunks past the end of the list are empty
    E = len(orc.visible_list(ctx - 1, ctx, w, G)[1])
    s = -(-E // S)
    for c in range(S):
        assert np.isfinite(lse[c]).all() == (c * s < E)


def test_split_merge_any_partition():
    ctx, w, G = 192, 40, 12
    q = rnd((1, 2, 8), 35)
    Kc, Vc = rnd((1, 1, ctx, 8), 36), rnd((1, 1, ctx, 8), 37)
    O1, L1 = orc.decode(q, Kc, Vc, w, G, 0.35)
    E = len(orc.visible_list(ctx - 1, ctx, w, G)[1])
    rng = np.random.default_rng(38)
    for _ in range(5):
        cuts = np.sort(rng.integers(0, E + 1, size=6))
        bnd = np.concatenate([[0], cuts, [E]])
        o, lse = orc.decode_partials(q, Kc, Vc, w, G, len(bnd) - 1, 0.35, bounds=bnd)
        O, L = orc.merge(o, lse)
        np.testing.assert_allclose(O, O1, atol=1e-13)
        np.testing.assert_allclose(L, L1, atol=1e-13)


@pytest.mark.parametrize("ctx,w,G", [(256, 64, 16), (128, 300, 8), (96, 5, 0)])
def test_decode_equals_prefill_last_row(ctx, w, G):
    Q = rnd((2, 4, ctx, 8), 39)
    Kc, Vc = rnd((2, 2, ctx, 8), 40), rnd((2, 2, ctx, 8), 41)
    O, L = orc.attn_dense(Q, Kc, Vc, w, G, 0.35)
    Od, Ld = orc.decode(Q[:, :, -1], Kc, Vc, w, G, 0.35)
    np.testing.assert_allclose(Od, O[:, :, -1], atol=1e-13)
    np.testing.assert_allclose(Ld, L[:, :, -1], atol=1e-13)


def test_visible_list_order_and_content():
    kinds, idx = orc.visible_list(i=99, n=100, w=30, G=10)
    # block b (positions 10b..10b+9) ends at or before 99-30=69: b <= 6
    assert list(idx[kinds == 0]) == list(range(7))
    assert list(idx[kinds == 1]) == list(range(70, 100))
    assert list(kinds) == [0] * 7 + [1] * 30


# ---------------------------------------------------------- sampled rows

def test_sampled_rows_match_dense():
    n, w, G = 512, 70, 16
    Q, K, V = rnd((1, 4, n, 8), 42), rnd((1, 2, n, 8), 43), rnd((1, 2, n, 8), 44)
    O, L = orc.attn_dense(Q, K, V, w, G, 0.3)
    rows = {h: np.sort(np.random.default_rng(h).choice(n, 50, replace=False)) for h in range(4)}
    res = orc.attn(Q, K, V, w, G, 0.3, rows=rows, group_span=37)
    for h, (r, o, l) in res.items():
        np.testing.assert_allclose(o, O[:, h, r], atol=1e-13)
        np.testing.assert_allclose(l, L[:, h, r], atol=1e-13)


# ---------------------------------------------------------- page figures

_PAIRS = {}


def pairs(n, w, G):
    """Visible pair counts from the oracle's predicates (cached: the 1M-row
    counts take several seconds)."""
    if (n, w, G) not in _PAIRS:
        _PAIRS[(n, w, G)] = orc.visible_pairs(n, w, G, chunk=512)
    return _PAIRS[(n, w, G)]


def test_page_cost_model_window_count():
    with open(os.path.join(GOLDEN, "page_figures.json")) as f:
        fig = json.load(f)["cost_model"]
    n, w, H = fig["tokens"], fig["window"], fig["heads"]
    win, _ = pairs(n, w, 0)
    total = H * win
    # the printed figure is tokens x window per head; the causal ramp at the
    # start (row i < w-1 sees only i+1 keys) is the exact difference
    assert total + H * w * (w - 1) // 2 == round(fig["window_dot_products"])
    assert abs(total - fig["window_dot_products"]) / fig["window_dot_products"] < w / n


def test_page_cost_model_landmark_bound():
    with open(os.path.join(GOLDEN, "page_figures.json")) as f:
        figs = json.load(f)
    fig, red = figs["cost_model"], figs["reduction"]
    n, w, G = red["tokens"], red["window"], red["landmarks"]
    win, lm = pairs(n, w, G)
    # every token sees at most all G landmarks; on the page that maximum is
    # the count (64 heads x 1M x 512 = 0.0328e12, printed 0.033e12)
    assert fig["heads"] * lm < fig["landmark_dot_products_exact"] * n / fig["tokens"]
    assert abs(fig["landmark_dot_products_exact"] - fig["landmark_dot_products_printed"]) < 0.5e9
    # roughly half the landmarks are visible on average (rows see blocks
    # entirely left of their window)
    assert 0.45 < lm / (n * G) < 0.5
    # O(n^2) -> O(n*w): n^2 / window pairs is the printed ~250x
    ratio = n * n / win
    assert abs(ratio - red["printed_reduction"]) / red["printed_reduction"] < 0.03


def test_page_block_sparse_fraction():
    with open(os.path.join(GOLDEN, "page_figures.json")) as f:
        fig = json.load(f)["block_sparse_fraction"]
    n, w = fig["tokens"], fig["window"]
    win, _ = pairs(n, w, 0)
    assert round(100 * win / n ** 2, 1) == fig["printed_percent"]
