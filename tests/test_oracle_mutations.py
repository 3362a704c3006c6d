"""Plant plausible mistakes in the oracle (on the CPU) and check that the
pins catch every one: a pin set that passes a broken oracle pins nothing."""
import numpy as np
import pytest

from oracle import msa_oracle as orc
from tests import test_oracle_backward as bwd
from tests import test_oracle_blocksparse as bsp
from tests import test_oracle_incremental as inc
from tests import test_oracle_pins as pins
from tests import test_oracle_plan_pins as plan


def _window_wide(i, j, w):          # w+1 keys
    return (np.asarray(j) <= np.asarray(i)) & (np.asarray(j) >= np.asarray(i) - w)


def _window_no_self(i, j, w):       # excludes the query's own key
    return (np.asarray(j) < np.asarray(i)) & (np.asarray(j) > np.asarray(i) - w - 1)


def _landmark_exclusive(i, b, L, w):   # block must end strictly before i - w
    return (np.asarray(b) + 1) * L - 1 < np.asarray(i) - w


def _landmark_straddle(i, b, L, w):    # block only has to start before i - w
    return np.asarray(b) * L <= np.asarray(i) - w


def _pool_sum(X, G):                   # sum instead of mean
    L = X.shape[-2] // G
    return orc.__dict__["_orig_pool"](X, G) * L


def _kv_head_mod(h, Hq, Hkv):          # interleaved instead of grouped
    return h % Hkv


def _softmax_drop_landmark_mass(S_win, M_win, S_lm, M_lm, V_span, V_lm):
    S_win = np.where(M_win, S_win, -np.inf)
    S_lm = np.where(M_lm, S_lm, -np.inf)
    m = np.maximum(S_win.max(axis=1, initial=-np.inf), S_lm.max(axis=1, initial=-np.inf))
    P_win = np.where(M_win, np.exp(S_win - m[:, None]), 0.0)
    P_lm = np.where(M_lm, np.exp(S_lm - m[:, None]), 0.0)
    l = P_win.sum(axis=1)                                  # landmark weights missing from l
    num = P_win @ V_span
    if V_lm is not None and V_lm.shape[0]:
        num = num + P_lm @ V_lm
    return num / l[:, None], m + np.log(l)


def _softmax_log2(S_win, M_win, S_lm, M_lm, V_span, V_lm):
    O, lse = orc.__dict__["_orig_softmax"](S_win, M_win, S_lm, M_lm, V_span, V_lm)
    return O, lse / np.log(2.0)                            # LSE in the wrong base


def _merge_unweighted(o, lse):
    fin = np.isfinite(lse)
    O = (o * fin[..., None]).sum(0) / fin.sum(0)[..., None]
    return O, orc.__dict__["_orig_merge"](o, lse)[1]


def _varlen_query_past_end(i, w, L, G_cap):   # decodes row n instead of n-1
    return orc.__dict__["_orig_vlf"](i + 1, w, L, G_cap)


def _pool_prefix_sum(X, n, L, G_cap):          # sum instead of mean
    return orc.__dict__["_orig_pool_prefix"](X, n, L, G_cap) * L


def _append_at_block_start(Kc, Vc, Kbar, Vbar, positions, k_new, v_new, L):
    # refreshes a landmark when its block's first row arrives, not its last
    for b, pos in enumerate(positions):
        pos = int(pos)
        if 0 <= pos < Kc.shape[2]:
            Kc[b, :, pos], Vc[b, :, pos] = k_new[b], v_new[b]
            if pos % L == 0:
                blk = pos // L
                Kbar[b, :, blk] = Kc[b, :, blk * L:(blk + 1) * L].mean(axis=1)
                Vbar[b, :, blk] = Vc[b, :, blk * L:(blk + 1) * L].mean(axis=1)


def _softmax_bwd_no_rowsum(P, dP, D):          # drops the D term
    return P * dP


def _mean_bwd_no_divide(dXbar, L):              # forgets the 1/L of the mean
    return np.repeat(dXbar, L, axis=-2)


def _mean_bwd_last_row(dXbar, L):               # sends the whole gradient to the block's last row
    out = np.zeros(dXbar.shape[:-2] + (dXbar.shape[-2] * L, dXbar.shape[-1]))
    out[..., L - 1::L, :] = dXbar
    return out


def _bs_mask_strict_causal(n, counts, indices, bq, bk, causal):   # causal without the diagonal
    M = orc.__dict__["_orig_bs_mask"](n, counts, indices, bq, bk, False)
    return np.tril(M, -1) if causal else M


def _bs_mask_block_short(n, counts, indices, bq, bk, causal):      # drops each block's last key
    M = orc.__dict__["_orig_bs_mask"](n, counts, indices, bq, bk, causal)
    M[:, bk - 1::bk] = 0
    return M


def _tile_plan_variant(interior_any=False, k_hi_short=False):
    """The oracle's tile enumeration with one planted mistake."""
    def tile_plan(n, w, G, BM, BN, q_tiles=None):
        T = -(-n // BM)
        ts = range(T) if q_tiles is None else q_tiles
        L = orc.block_len(n, G) if G else 0
        out = []
        for t in ts:
            rws = np.arange(t * BM, min(n, t * BM + BM))
            if G:
                for lt in range(-(-G // BN)):
                    b = np.arange(lt * BN, lt * BN + BN)
                    M = orc.landmark_visible(rws[:, None], b[None, :], L, w) & (b[None, :] < G)
                    if M.any():
                        out.append((t, 0, lt, bool(M.any() if interior_any else M.all())))
            k_lo = max(0, int(rws[0]) - w) // BN
            k_hi = min(-(-n // BN) - 1, (int(rws[-1]) + 1) // BN)
            if k_hi_short:
                k_hi = (int(rws[-1])) // BN - 1
            for kt in range(k_lo, k_hi + 1):
                j = np.arange(kt * BN, kt * BN + BN)
                M = orc.window_visible(rws[:, None], j[None, :], w) & (j[None, :] < n)
                if M.any():
                    out.append((t, 1, kt, bool(M.any() if interior_any else M.all())))
        return out
    return tile_plan


def _row_plan_lo_from_top(n, w, G, rows=None):     # lowest visible key read from the wrong end
    lo, cnt = orc.__dict__["_orig_row_plan"](n, w, G, rows)
    r = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    return np.where(r - lo + 1 > 1, r, lo), cnt


def _bwd_ignores_given_output(Q, K, V, dO, w, G, scale=None, kv_heads=None, group_span=512, O=None):
    # forms D from the exact forward output even when handed another one
    return orc.__dict__["_orig_attn_bwd"](Q, K, V, dO, w, G, scale, kv_heads, group_span)


def _chunk_bounds_floor(E, S):                     # floor(E/S) entries per chunk
    s = E // S
    return np.array([min(E, c * s) for c in range(S)] + [E], dtype=np.int64)


MUTANTS = {
    "window_wide": ("window_visible", _window_wide),
    "window_no_self": ("window_visible", _window_no_self),
    "landmark_exclusive": ("landmark_visible", _landmark_exclusive),
    "landmark_straddle": ("landmark_visible", _landmark_straddle),
    "pool_sum": ("pool", _pool_sum),
    "kv_head_mod": ("kv_head", _kv_head_mod),
    "softmax_drop_landmark_mass": ("_softmax_rows", _softmax_drop_landmark_mass),
    "lse_log2": ("_softmax_rows", _softmax_log2),
    "merge_unweighted": ("merge", _merge_unweighted),
    "varlen_query_past_end": ("visible_list_fixed", _varlen_query_past_end),
    "pool_prefix_sum": ("pool_prefix", _pool_prefix_sum),
    "append_at_block_start": ("append_tokens", _append_at_block_start),
    "bwd_no_rowsum": ("_softmax_bwd", _softmax_bwd_no_rowsum),
    "bwd_mean_no_divide": ("_mean_bwd", _mean_bwd_no_divide),
    "bwd_mean_last_row": ("_mean_bwd", _mean_bwd_last_row),
    "bs_strict_causal": ("blocksparse_mask", _bs_mask_strict_causal),
    "bs_block_short": ("blocksparse_mask", _bs_mask_block_short),
    "tile_interior_any": ("tile_plan", _tile_plan_variant(interior_any=True)),
    "tile_k_hi_short": ("tile_plan", _tile_plan_variant(k_hi_short=True)),
    "row_plan_lo_from_top": ("row_plan", _row_plan_lo_from_top),
    "chunk_bounds_floor": ("chunk_bounds", _chunk_bounds_floor),
    "bwd_ignores_given_output": ("attn_bwd", _bwd_ignores_given_output),
}

PIN_SET = [
    lambda: pins.test_brute_force_mha(16, 3, 4),
    lambda: pins.test_brute_force_gqa_batch(16, 3, 4),
    lambda: pins.test_full_window_no_landmarks_is_causal_sdpa(64, 64),
    lambda: pins.test_one_token_landmarks_give_causal_attention_for_any_window(7),
    lambda: pins.test_golden_uniform_worked_example(),
    lambda: pins.test_zero_keys_average_the_visible_values(128, 16, 8),
    lambda: pins.test_key_shift_moves_lse_only(),
    lambda: pins.test_pool_constant_blocks_and_bruteforce(),
    lambda: pins.test_split_merge_any_partition(),
    lambda: pins.test_decode_equals_prefill_last_row(256, 64, 16),
    lambda: pins.test_window_one_no_landmarks_is_identity(),
    lambda: inc.test_varlen_equals_prefill_row_of_padded_sequence(17, 3, 4),
    lambda: inc.test_varlen_window_covers_everything_is_textbook_causal(9),
    lambda: inc.test_append_builds_closed_form_landmarks(),
    lambda: inc.test_append_then_decode_equals_decode_of_the_whole_prefix(),
    lambda: bwd.test_backward_matches_finite_differences(9, 4, 3),
    lambda: bwd.test_one_token_landmarks_give_causal_backward(7),
    lambda: bsp.test_full_causal_lists_are_causal_sdpa(),
    lambda: bsp.test_brute_force_random_lists(True),
    lambda: plan.test_tile_plan_equals_brute_force(130, 65, 10, 64, 64),
    lambda: plan.test_row_plan_equals_brute_force(300, 63, 10),
    lambda: plan.test_chunk_bounds_decode_workload(),
    lambda: plan.test_chunk_bounds_with_empty_chunks(),
    lambda: bwd.test_given_output_enters_through_d_only(64, 9, 8),
]


def _failures():
    n = 0
    for pin in PIN_SET:
        try:
            pin()
        except Exception:  # a wrong value or a crash: either way the pin caught it
            n += 1
    return n


def test_unmutated_oracle_passes_the_pin_set():
    assert _failures() == 0


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setitem(orc.__dict__, "_orig_pool", orc.pool)
    monkeypatch.setitem(orc.__dict__, "_orig_softmax", orc._softmax_rows)
    monkeypatch.setitem(orc.__dict__, "_orig_merge", orc.merge)
    monkeypatch.setitem(orc.__dict__, "_orig_vlf", orc.visible_list_fixed)
    monkeypatch.setitem(orc.__dict__, "_orig_pool_prefix", orc.pool_prefix)
    monkeypatch.setitem(orc.__dict__, "_orig_bs_mask", orc.blocksparse_mask)
    monkeypatch.setitem(orc.__dict__, "_orig_row_plan", orc.row_plan)
    monkeypatch.setitem(orc.__dict__, "_orig_attn_bwd", orc.attn_bwd)
    monkeypatch.setattr(orc, attr, fn)
    assert _failures() > 0, f"no pin caught the planted mistake {name}"
