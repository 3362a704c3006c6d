"""Pins of the oracle's backward (gradients of O with respect to Q, K, V)
against facts fixed outside it: central finite differences of the already
pinned forward, torch autograd of textbook causal attention where the
pattern reduces to it, GQA as MHA with repeated K/V, and closed forms."""
import numpy as np
import pytest
import torch

from oracle import msa_oracle as orc

SC = 0.4


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def finite_diff(Q, K, V, dO, w, G, scale, h=1e-6):
    """Central differences of sum(dO * O) with respect to every input element."""
    def loss(args):
        O, _ = orc.attn_dense(*args, w, G, scale)
        return float((O * dO).sum())
    grads = []
    for idx in range(3):
        X = (Q, K, V)[idx]
        g = np.zeros_like(X)
        for ix in np.ndindex(X.shape):
            args = [Q, K, V]
            Xp, Xm = X.copy(), X.copy()
            Xp[ix] += h
            Xm[ix] -= h
            args[idx] = Xp
            lp = loss(args)
            args[idx] = Xm
            lm = loss(args)
            g[ix] = (lp - lm) / (2 * h)
        grads.append(g)
    return grads


FD_CASES = [(12, 3, 4), (12, 12, 0), (12, 2, 2), (12, 5, 12), (12, 1, 3), (9, 4, 3), (8, 20, 1)]


@pytest.mark.parametrize("n,w,G", FD_CASES)
def test_backward_matches_finite_differences(n, w, G):
    B, Hq, Hkv, d = 2, 4, 2, 3
    Q, K, V = rnd((B, Hq, n, d), n), rnd((B, Hkv, n, d), n + 1), rnd((B, Hkv, n, d), n + 2)
    dO = rnd((B, Hq, n, d), n + 3)
    got = orc.attn_bwd(Q, K, V, dO, w, G, SC)
    want = finite_diff(Q, K, V, dO, w, G, SC)
    for name, a, b in zip("QKV", got, want):
        np.testing.assert_allclose(a, b, atol=2e-8 * max(1.0, np.abs(b).max()), err_msg=f"d{name}")


def torch_causal_grads(Q, K, V, dO, scale):
    t = [torch.tensor(x, requires_grad=True) for x in (Q, K, V)]
    O = torch.nn.functional.scaled_dot_product_attention(*t, is_causal=True, scale=scale)
    O.backward(torch.tensor(dO))
    return [x.grad.numpy() for x in t]


@pytest.mark.parametrize("n,w", [(64, 64), (48, 100)])
def test_full_window_no_landmarks_is_causal_sdpa_backward(n, w):
    Q, K, V, dO = (rnd((1, 3, n, 8), s) for s in (60, 61, 62, 63))
    got = orc.attn_bwd(Q, K, V, dO, w, 0, SC)
    want = torch_causal_grads(Q, K, V, dO, SC)
    for a, b in zip(got, want):
        np.testing.assert_allclose(a, b, atol=1e-12)


@pytest.mark.parametrize("w", [1, 2, 7, 30])
def test_one_token_landmarks_give_causal_backward(w):
    # G = n: landmark j is key j itself; window + visible landmarks cover
    # every j <= i exactly once, so the gradients (through the window and
    # through the mean of a one-row block) are those of causal attention
    n = 40
    Q, K, V, dO = (rnd((1, 2, n, 8), s) for s in (70, 71, 72, 73))
    got = orc.attn_bwd(Q, K, V, dO, w, n, SC)
    want = torch_causal_grads(Q, K, V, dO, SC)
    for a, b in zip(got, want):
        np.testing.assert_allclose(a, b, atol=1e-12)


def test_gqa_backward_equals_mha_with_repeated_kv():
    n, w, G = 64, 9, 8
    Q, dO = rnd((1, 6, n, 8), 80), rnd((1, 6, n, 8), 81)
    K, V = rnd((1, 2, n, 8), 82), rnd((1, 2, n, 8), 83)
    dQ, dK, dV = orc.attn_bwd(Q, K, V, dO, w, G, SC)
    Kr, Vr = np.repeat(K, 3, axis=1), np.repeat(V, 3, axis=1)
    dQm, dKm, dVm = orc.attn_bwd(Q, Kr, Vr, dO, w, G, SC)
    np.testing.assert_allclose(dQ, dQm, atol=1e-12)
    np.testing.assert_allclose(dK, dKm.reshape(1, 2, 3, n, 8).sum(2), atol=1e-12)
    np.testing.assert_allclose(dV, dVm.reshape(1, 2, 3, n, 8).sum(2), atol=1e-12)


def test_constant_values_give_zero_query_and_key_gradients():
    # every visible value equal: O is that value whatever the scores, so
    # nothing flows to Q or K; dV sums to sum(dO) per row (P sums to 1)
    n, w, G = 64, 7, 8
    Q, K, dO = rnd((1, 2, n, 8), 90), rnd((1, 2, n, 8), 91), rnd((1, 2, n, 8), 92)
    V = np.broadcast_to(rnd((8,), 93), (1, 2, n, 8)).copy()
    dQ, dK, dV = orc.attn_bwd(Q, K, V, dO, w, G, SC)
    assert np.abs(dQ).max() < 1e-12 and np.abs(dK).max() < 1e-12
    np.testing.assert_allclose(dV.sum(axis=2), dO.sum(axis=2), atol=1e-12)


def test_dq_rows_equal_full_dq():
    n, w, G = 256, 20, 16
    Q, K, V, dO = rnd((2, 4, n, 8), 100), rnd((2, 2, n, 8), 101), rnd((2, 2, n, 8), 102), rnd((2, 4, n, 8), 103)
    dQ, _, _ = orc.attn_bwd(Q, K, V, dO, w, G, SC, group_span=37)
    rows = {h: np.sort(np.random.default_rng(h).choice(n, 40, replace=False)) for h in (0, 3)}
    res = orc.attn_bwd_dq_rows(Q, K, V, dO, w, G, SC, rows=rows, group_span=50)
    for h, (r, dq) in res.items():
        np.testing.assert_allclose(dq, dQ[:, h, r], atol=1e-12)


def test_kv_head_subset_matches_full():
    n, w, G = 128, 10, 8
    Q, K, V, dO = rnd((1, 4, n, 8), 110), rnd((1, 2, n, 8), 111), rnd((1, 2, n, 8), 112), rnd((1, 4, n, 8), 113)
    full = orc.attn_bwd(Q, K, V, dO, w, G, SC)
    part = orc.attn_bwd(Q, K, V, dO, w, G, SC, kv_heads=[1])
    np.testing.assert_allclose(part[0][:, 2:], full[0][:, 2:], atol=1e-13)
    np.testing.assert_allclose(part[1][:, 1], full[1][:, 1], atol=1e-13)
    np.testing.assert_allclose(part[2][:, 1], full[2][:, 1], atol=1e-13)
    assert not part[0][:, :2].any() and not part[1][:, 0].any()


@pytest.mark.parametrize("n,w,G", [(64, 9, 8), (40, 100, 0), (48, 5, 48)])
def test_given_output_enters_through_d_only(n, w, G):
    # The backward handed O + delta instead of the exact O changes the softmax
    # term D_i = dO_i . O_i by dD_i = dO_i . delta_i and nothing else.  From
    # dS = P (dP - D): dQ_i moves by -scale dD_i (P K)_i, where (P K)_i is the
    # forward run with K as the values (landmarks of K are the key
    # landmarks); dK moves by -scale times the value gradient that the
    # upstream gradient dD_i q_i would give (dV = P^T dO has the same form,
    # window and landmark scatter included); dV does not move.
    B, Hq, Hkv, d = 2, 4, 2, 8
    Q, K, V = rnd((B, Hq, n, d), 120), rnd((B, Hkv, n, d), 121), rnd((B, Hkv, n, d), 122)
    dO, delta = rnd((B, Hq, n, d), 123), 1e-3 * rnd((B, Hq, n, d), 124)
    O_exact, _ = orc.attn_dense(Q, K, V, w, G, SC)
    base = orc.attn_bwd(Q, K, V, dO, w, G, SC)
    same = orc.attn_bwd(Q, K, V, dO, w, G, SC, O=O_exact)
    for a, b in zip(base, same):
        np.testing.assert_allclose(a, b, atol=1e-13)
    dQ1, dK1, dV1 = orc.attn_bwd(Q, K, V, dO, w, G, SC, O=O_exact + delta)
    dD = (dO * delta).sum(axis=-1, keepdims=True)
    PK, _ = orc.attn_dense(Q, K, K, w, G, SC)
    np.testing.assert_allclose(dQ1 - base[0], -SC * dD * PK, atol=1e-13)
    _, _, dV_of_dDq = orc.attn_bwd(Q, K, V, dD * Q, w, G, SC)
    np.testing.assert_allclose(dK1 - base[1], -SC * dV_of_dDq, atol=1e-13)
    np.testing.assert_allclose(dV1, base[2], atol=1e-13)
    # the sampled-rows dQ takes the same given output on its rows
    rows = {h: np.sort(np.random.default_rng(h).choice(n, 12, replace=False)) for h in (1, 2)}
    Og = {h: (O_exact + delta)[:, h, r] for h, r in rows.items()}
    for h, (r, dq) in orc.attn_bwd_dq_rows(Q, K, V, dO, w, G, SC, rows=rows, O=Og).items():
        np.testing.assert_allclose(dq, dQ1[:, h, r], atol=1e-13)
