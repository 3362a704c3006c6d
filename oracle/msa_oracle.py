"""fp64 CPU oracle for causal sliding-window + mean-pooled-landmark attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package may import, call or
execute this module; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path: it uses numpy only.

What is computed (the pattern the pages call Flash-MSA, made precise):

* "Scaling GPU Cluster for Million Token Context", section "Why Sparse
  Attention Changes the Game": each query attends to a local window of
  recent tokens plus a small set of landmark tokens that summarise distant
  context; section "What is Flash-MSA Sparse Attention in GPU Clusters?":
  both parts are computed in one fused pass.
* "Training at 1M+ Token Context ...", Block-Sparse Flash Attention
  paragraph: distant context is represented by compression tokens, local
  tokens by a sliding window.

Readings taken where the pages leave the step open:

* A landmark b is the plain mean of K and V over block b of L = n / G
  consecutive positions (no learned projection).
* Query i sees key j iff i - w < j <= i (w keys including itself, clipped at
  position 0), and sees landmark b iff the block's last position
  (b+1)*L - 1 is at or before i - w.  Blocks that straddle the window edge
  are not visible.
* Window keys and visible landmarks share ONE softmax with one scale
  (1/sqrt(d) by default); the output is O_i and LSE_i = m_i + ln(l_i) with
  the natural log, in units of the scaled score.
* Query head h reads KV head h // (Hq / Hkv).
* Decode is the same computation for the single row i = ctx - 1.  The
  split form partitions the ordered visible list (landmarks ascending, then
  window keys ascending) into S contiguous chunks of ceil(E / S) entries and
  merges the per-chunk results by their log-sum-exp, which is the one-GPU
  form of the softmax-statistics aggregation in the Ring Attention paragraph
  of the "Training at 1M+ Token Context" page.

* Incremental decode (sequences of different lengths in one cache, one
  token appended per step): the block length L is fixed by the cache's
  capacity, a landmark is the mean of its block once all L rows are in the
  cache, and the visibility rule is unchanged, so a visible landmark is
  always a complete block.  With every length equal to the capacity this is
  the decode above.  A sequence of length 0 has O = 0 and LSE = -inf.

* Backward: the gradients of O with respect to Q, K and V for an upstream
  dO are the chain rule through the same single softmax; a landmark is the
  mean of its block, so each row of the block receives 1/L of the
  landmark's gradient.  The pages train at these lengths but do not write
  the backward out.

* Block-sparse lists: each query block sees the keys of the key blocks
  listed for it (optionally causal), one softmax; see Step 9.

Every predicate below is evaluated by explicit comparisons; nothing uses a
closed-form count of visible keys.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

NEG_INF = -np.inf


# ---------------------------------------------------------------------------
# Step 1: landmarks (mean of each block of L = n / G positions)
# ---------------------------------------------------------------------------

def block_len(n: int, G: int) -> int:
    """Block length L = n / G.  G must divide n."""
    if G <= 0:
        raise ValueError("no landmarks: G must be > 0 to have a block length")
    if n % G:
        raise ValueError(f"G={G} does not divide n={n}")
    return n // G


def pool(X: np.ndarray, G: int) -> np.ndarray:
    """Landmarks of X [..., n, d]: [..., G, d], entry b = mean of rows
    b*L .. b*L+L-1, in fp64."""
    n = X.shape[-2]
    L = block_len(n, G)
    Xd = np.asarray(X, dtype=np.float64)
    out = np.empty(Xd.shape[:-2] + (G, Xd.shape[-1]), dtype=np.float64)
    for b in range(G):
        out[..., b, :] = Xd[..., b * L:(b + 1) * L, :].mean(axis=-2)
    return out


# ---------------------------------------------------------------------------
# Step 2: visibility predicates (explicit comparisons)
# ---------------------------------------------------------------------------

def window_visible(i, j, w: int):
    """Key j lies in query i's causal window: i - w < j <= i."""
    i = np.asarray(i)
    j = np.asarray(j)
    return (j <= i) & (j > i - w)


def landmark_visible(i, b, L: int, w: int):
    """Landmark b (positions b*L .. (b+1)*L-1) ends at or before i - w."""
    i = np.asarray(i)
    b = np.asarray(b)
    return (b + 1) * L - 1 <= i - w


def dense_masks(n: int, w: int, G: int) -> Tuple[np.ndarray, np.ndarray]:
    """Full boolean masks M_win [n, n] and M_lm [n, G] (small n only)."""
    i = np.arange(n)[:, None]
    m_win = window_visible(i, np.arange(n)[None, :], w)
    if G:
        m_lm = landmark_visible(i, np.arange(G)[None, :], block_len(n, G), w)
    else:
        m_lm = np.zeros((n, 0), dtype=bool)
    return m_win, m_lm


def kv_head(h: int, Hq: int, Hkv: int) -> int:
    """KV head read by query head h: consecutive groups of Hq / Hkv."""
    return h // (Hq // Hkv)


# ---------------------------------------------------------------------------
# Steps 3-4: scores, one softmax over the union, output and LSE
# ---------------------------------------------------------------------------

def _softmax_rows(S_win, M_win, S_lm, M_lm, V_span, V_lm):
    """One softmax per row over the visible window scores and the visible
    landmark scores together.  Returns (O [R, d], LSE [R])."""
    S_win = np.where(M_win, S_win, NEG_INF)
    S_lm = np.where(M_lm, S_lm, NEG_INF)
    m = np.maximum(S_win.max(axis=1, initial=NEG_INF), S_lm.max(axis=1, initial=NEG_INF))
    P_win = np.where(M_win, np.exp(S_win - m[:, None]), 0.0)
    P_lm = np.where(M_lm, np.exp(S_lm - m[:, None]), 0.0)
    l = P_win.sum(axis=1) + P_lm.sum(axis=1)
    num = P_win @ V_span
    if V_lm is not None and V_lm.shape[0]:
        num = num + P_lm @ V_lm
    O = num / l[:, None]
    lse = m + np.log(l)
    return O, lse


def _row_groups(rows: np.ndarray, span: int) -> List[np.ndarray]:
    """Split sorted rows into consecutive groups covering at most `span`
    positions each (so that each group's key range stays small)."""
    groups = []
    start = 0
    for k in range(1, len(rows) + 1):
        if k == len(rows) or rows[k] - rows[start] >= span:
            groups.append(rows[start:k])
            start = k
    return groups


def attn(Q, K, V, w: int, G: int, scale: Optional[float] = None,
         rows: Optional[Dict[int, np.ndarray]] = None,
         Kbar: Optional[np.ndarray] = None, Vbar: Optional[np.ndarray] = None,
         group_span: int = 512):
    """Window + landmark attention, fp64.

    Q [B, Hq, n, d]; K, V [B, Hkv, n, d].  ``rows`` maps a query head to the
    sorted query rows to evaluate (default: every row of every head).  Kbar
    and Vbar may be given (e.g. to feed landmarks pooled elsewhere);
    otherwise they are the fp64 means of K and V.

    Returns {head: (rows, O [B, R, d], LSE [B, R])}.

    For each group of nearby rows the scores are formed against every key in
    a range that strictly contains the rows' windows (one extra key of margin
    on each side), and the window predicate decides visibility of each of
    them; the landmark predicate is evaluated against every landmark.
    """
    if w < 1:
        raise ValueError("window must be >= 1")
    Q = np.asarray(Q)
    B, Hq, n, d = Q.shape
    Hkv = K.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if G:
        L = block_len(n, G)
        if Kbar is None:
            Kbar = pool(K, G)
        if Vbar is None:
            Vbar = pool(V, G)
    results = {}
    heads = range(Hq) if rows is None else sorted(rows)
    for h in heads:
        g = kv_head(h, Hq, Hkv)
        r_all = np.arange(n) if rows is None else np.asarray(rows[h], dtype=np.int64)
        O = np.empty((B, len(r_all), d))
        LSE = np.empty((B, len(r_all)))
        pos = 0
        for grp_rows in _row_groups(r_all, group_span):
            lo = max(0, int(grp_rows[0]) - w)           # one below the lowest visible key
            hi = min(n, int(grp_rows[-1]) + 2)          # one above the highest visible key
            keys = np.arange(lo, hi)
            M_win = window_visible(grp_rows[:, None], keys[None, :], w)
            if G:
                M_lm = landmark_visible(grp_rows[:, None], np.arange(G)[None, :], L, w)
            for b in range(B):
                q = np.asarray(Q[b, h, grp_rows], dtype=np.float64)
                k_span = np.asarray(K[b, g, lo:hi], dtype=np.float64)
                v_span = np.asarray(V[b, g, lo:hi], dtype=np.float64)
                S_win = scale * (q @ k_span.T)
                if G:
                    kb = np.asarray(Kbar[b, g], dtype=np.float64)
                    vb = np.asarray(Vbar[b, g], dtype=np.float64)
                    S_lm = scale * (q @ kb.T)
                    o, lse = _softmax_rows(S_win, M_win, S_lm, M_lm, v_span, vb)
                else:
                    empty = np.zeros((len(grp_rows), 0))
                    o, lse = _softmax_rows(S_win, M_win, empty, empty.astype(bool), v_span, None)
                O[b, pos:pos + len(grp_rows)] = o
                LSE[b, pos:pos + len(grp_rows)] = lse
            pos += len(grp_rows)
        results[h] = (r_all, O, LSE)
    return results


def attn_dense(Q, K, V, w: int, G: int, scale: Optional[float] = None):
    """All rows: O [B, Hq, n, d], LSE [B, Hq, n] (small n)."""
    B, Hq, n, d = np.asarray(Q).shape
    res = attn(Q, K, V, w, G, scale)
    O = np.stack([res[h][1] for h in range(Hq)], axis=1)
    LSE = np.stack([res[h][2] for h in range(Hq)], axis=1)
    return O, LSE


# ---------------------------------------------------------------------------
# Step 5: integer artefacts derived from the masks
# ---------------------------------------------------------------------------

def row_plan(n: int, w: int, G: int, rows: Optional[np.ndarray] = None):
    """For each row: the lowest visible window key and the number of visible
    landmarks, both read off the explicit predicates.  Returns (win_lo,
    lm_count) as int64 arrays over ``rows`` (default all rows)."""
    r = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    win_lo = np.empty(len(r), dtype=np.int64)
    lm_count = np.zeros(len(r), dtype=np.int64)
    L = block_len(n, G) if G else 0
    for s in range(0, len(r), 256):
        rr = r[s:s + 256]
        lo = max(0, int(rr.min()) - w)
        keys = np.arange(lo, min(n, int(rr.max()) + 2))
        M = window_visible(rr[:, None], keys[None, :], w)
        win_lo[s:s + 256] = keys[np.argmax(M, axis=1)]
        if G:
            lm_count[s:s + 256] = landmark_visible(rr[:, None], np.arange(G)[None, :], L, w).sum(axis=1)
    return win_lo, lm_count


def tile_plan(n: int, w: int, G: int, BM: int, BN: int, q_tiles: Optional[Sequence[int]] = None):
    """The block-sparse tile set for query tiles of BM rows and key tiles of
    BN keys, read off the masks: a (query tile, key tile) pair is listed iff
    some (row, key) in it is visible, and flagged interior iff every slot of
    it is visible (slots past the last key or landmark count as invisible).

    Returns a list of (t, kind, tile, interior) with kind 0 = landmark tile,
    1 = window tile, ordered by t, then kind, then tile."""
    T = -(-n // BM)
    ts = range(T) if q_tiles is None else q_tiles
    L = block_len(n, G) if G else 0
    out = []
    for t in ts:
        rws = np.arange(t * BM, min(n, t * BM + BM))
        if G:
            for lt in range(-(-G // BN)):
                b = np.arange(lt * BN, lt * BN + BN)
                M = landmark_visible(rws[:, None], b[None, :], L, w) & (b[None, :] < G)
                if M.any():
                    out.append((t, 0, lt, bool(M.all())))
        # candidate key tiles: those overlapping [first row - w, last row + 1]
        k_lo = max(0, int(rws[0]) - w) // BN
        k_hi = min(-(-n // BN) - 1, (int(rws[-1]) + 1) // BN)
        for kt in range(k_lo, k_hi + 1):
            j = np.arange(kt * BN, kt * BN + BN)
            M = window_visible(rws[:, None], j[None, :], w) & (j[None, :] < n)
            if M.any():
                out.append((t, 1, kt, bool(M.all())))
    return out


def visible_pairs(n: int, w: int, G: int, chunk: int = 4096) -> Tuple[int, int]:
    """Total visible (query, key) window pairs and (query, landmark) pairs
    of one head, counted from the predicates."""
    L = block_len(n, G) if G else 0
    win = 0
    lm = 0
    for s in range(0, n, chunk):
        rr = np.arange(s, min(n, s + chunk))
        lo = max(0, s - w)
        keys = np.arange(lo, min(n, int(rr[-1]) + 2))
        win += int(window_visible(rr[:, None], keys[None, :], w).sum())
        if G:
            lm += int(landmark_visible(rr[:, None], np.arange(G)[None, :], L, w).sum())
    return win, lm


# ---------------------------------------------------------------------------
# Step 6: decode (single row i = ctx-1) and its split / LSE-merge form
# ---------------------------------------------------------------------------

def visible_list(i: int, n: int, w: int, G: int) -> Tuple[np.ndarray, np.ndarray]:
    """Ordered visible entries of row i: the visible landmarks in block
    order, then the visible window keys ascending.  Returns (kinds, idx):
    kind 0 = landmark index, 1 = key position."""
    L = block_len(n, G) if G else 0
    lm = np.arange(G)
    lm = lm[landmark_visible(i, lm, L, w)] if G else lm
    keys = np.arange(max(0, i - w), min(n, i + 2))
    keys = keys[window_visible(i, keys, w)]
    kinds = np.concatenate([np.zeros(len(lm), np.int64), np.ones(len(keys), np.int64)])
    return kinds, np.concatenate([lm, keys]).astype(np.int64)


def chunk_bounds(E: int, S: int) -> np.ndarray:
    """Chunk c covers entries [c*s, min(E, (c+1)*s)) with s = ceil(E/S)."""
    s = -(-E // S) if E else 0
    return np.array([min(E, c * s) for c in range(S + 1)], dtype=np.int64)


def _entries(q, kc, vc, kb, vb, kinds, idx, scale):
    """Scores and values of the listed entries for one (sequence, head)."""
    d = q.shape[-1]
    kmat = np.empty((len(idx), d))
    vmat = np.empty((len(idx), d))
    is_lm = kinds == 0
    kmat[is_lm] = kb[idx[is_lm]]
    vmat[is_lm] = vb[idx[is_lm]]
    kmat[~is_lm] = kc[idx[~is_lm]]
    vmat[~is_lm] = vc[idx[~is_lm]]
    return scale * (kmat @ q), vmat


def decode_partials(q, Kc, Vc, w: int, G: int, S: int, scale: Optional[float] = None,
                    Kbar=None, Vbar=None, bounds: Optional[np.ndarray] = None):
    """Per-chunk results of decode.  q [B, Hq, d], caches [B, Hkv, ctx, d].
    Returns (o [S, B, Hq, d], lse [S, B, Hq]); an empty chunk has lse = -inf
    and o = 0.  ``bounds`` overrides the chunk boundaries (length S+1)."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv, ctx = Kc.shape[1], Kc.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if G:
        Kbar = pool(Kc, G) if Kbar is None else Kbar
        Vbar = pool(Vc, G) if Vbar is None else Vbar
    i = ctx - 1
    kinds, idx = visible_list(i, ctx, w, G)
    E = len(idx)
    bnd = chunk_bounds(E, S) if bounds is None else np.asarray(bounds)
    o = np.zeros((S, B, Hq, d))
    lse = np.full((S, B, Hq), NEG_INF)
    for b in range(B):
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            kb = np.asarray(Kbar[b, g], np.float64) if G else np.zeros((0, d))
            vb = np.asarray(Vbar[b, g], np.float64) if G else np.zeros((0, d))
            s_all, v_all = _entries(q[b, h], np.asarray(Kc[b, g], np.float64),
                                    np.asarray(Vc[b, g], np.float64), kb, vb, kinds, idx, scale)
            for c in range(S):
                a, e = int(bnd[c]), int(bnd[c + 1])
                if e <= a:
                    continue
                s = s_all[a:e]
                m = s.max()
                p = np.exp(s - m)
                l = p.sum()
                o[c, b, h] = (p @ v_all[a:e]) / l
                lse[c, b, h] = m + np.log(l)
    return o, lse


def merge(o: np.ndarray, lse: np.ndarray):
    """Combine chunk results: LSE = ln sum_c exp(lse_c), O = sum_c
    exp(lse_c - LSE) o_c.  Empty chunks (lse_c = -inf) get weight 0."""
    m = lse.max(axis=0)
    wts = np.where(np.isfinite(lse), np.exp(lse - m), 0.0)
    tot = wts.sum(axis=0)
    LSE = m + np.log(tot)
    O = (wts[..., None] * o).sum(axis=0) / tot[..., None]
    return O, LSE


def decode(q, Kc, Vc, w: int, G: int, scale: Optional[float] = None, Kbar=None, Vbar=None):
    """Unsplit decode: one softmax over every visible entry of row ctx-1.
    Returns (O [B, Hq, d], LSE [B, Hq])."""
    o, lse = decode_partials(q, Kc, Vc, w, G, 1, scale, Kbar, Vbar)
    return o[0], lse[0]


# ---------------------------------------------------------------------------
# Step 7: incremental decode -- sequences of different lengths that grow one
# token at a time ("Million Token Context Window Optimization: What Actually
# Works", section "Flash MSA vs Flash Attention: The real difference":
# generation continues after the long prompt; section "Benchmarking your
# optimization": the KV cache is the per-token state).  Reading where the
# pages are silent: the landmark block length L is fixed; landmark b is the
# mean of rows bL .. bL+L-1 and exists once that block is complete; the
# visibility rule is the one above, so a visible landmark is always a
# complete block.  With every length equal to G*L this is decode() above.
# ---------------------------------------------------------------------------

def pool_prefix(X, n: int, L: int, G_cap: int):
    """Landmarks of the first n rows of X [B, H, >=n, d] with block length L:
    [B, H, G_cap, d], complete blocks b < n // L hold the block mean (fp64),
    the others are zero (they are never visible)."""
    X = np.asarray(X, dtype=np.float64)
    B, H, _, d = X.shape
    out = np.zeros((B, H, G_cap, d))
    nb = min(n // L, G_cap)
    if nb:
        out[:, :, :nb] = X[:, :, :nb * L].reshape(B, H, nb, L, d).mean(axis=3)
    return out


def visible_list_fixed(i: int, w: int, L: int, G_cap: int) -> Tuple[np.ndarray, np.ndarray]:
    """Ordered visible entries of row i with fixed block length L: landmarks
    b < G_cap with (b+1)*L - 1 <= i - w in block order, then the window keys
    i-w < j <= i ascending.  Returns (kinds, idx) as visible_list()."""
    lm = np.arange(G_cap)
    lm = lm[landmark_visible(i, lm, L, w)] if G_cap else lm
    keys = np.arange(max(0, i - w), i + 1)
    keys = keys[window_visible(i, keys, w)]
    kinds = np.concatenate([np.zeros(len(lm), np.int64), np.ones(len(keys), np.int64)])
    return kinds, np.concatenate([lm, keys]).astype(np.int64)


def decode_varlen_partials(q, Kc, Vc, ctx_lens, w: int, L: int, G_cap: int, S: int,
                           scale: Optional[float] = None, Kbar=None, Vbar=None):
    """Per-chunk decode results when sequence b holds ctx_lens[b] tokens of a
    cache [B, Hkv, C, d] (query position ctx_lens[b]-1), landmark blocks of
    fixed length L.  Landmarks are pooled from each sequence's own prefix
    unless given ([B, Hkv, G_cap, d]).  Chunking per sequence as in
    chunk_bounds().  Returns (o [S, B, Hq, d], lse [S, B, Hq])."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = Kc.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = np.zeros((S, B, Hq, d))
    lse = np.full((S, B, Hq), NEG_INF)
    for b in range(B):
        n = int(ctx_lens[b])
        kinds, idx = visible_list_fixed(n - 1, w, L, G_cap)
        bnd = chunk_bounds(len(idx), S)
        kc_b = np.asarray(Kc[b:b + 1, :, :n], np.float64)
        vc_b = np.asarray(Vc[b:b + 1, :, :n], np.float64)
        kb_b = pool_prefix(kc_b, n, L, G_cap)[0] if Kbar is None else np.asarray(Kbar[b], np.float64)
        vb_b = pool_prefix(vc_b, n, L, G_cap)[0] if Vbar is None else np.asarray(Vbar[b], np.float64)
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            s_all, v_all = _entries(q[b, h], kc_b[0, g], vc_b[0, g], kb_b[g], vb_b[g], kinds, idx, scale)
            for c in range(S):
                a, e = int(bnd[c]), int(bnd[c + 1])
                if e <= a:
                    continue
                sc = s_all[a:e]
                m = sc.max()
                p = np.exp(sc - m)
                l = p.sum()
                o[c, b, h] = (p @ v_all[a:e]) / l
                lse[c, b, h] = m + np.log(l)
    return o, lse


def decode_varlen(q, Kc, Vc, ctx_lens, w: int, L: int, G_cap: int, scale: Optional[float] = None,
                  Kbar=None, Vbar=None):
    """Unsplit incremental decode.  Returns (O [B, Hq, d], LSE [B, Hq])."""
    o, lse = decode_varlen_partials(q, Kc, Vc, ctx_lens, w, L, G_cap, 1, scale, Kbar, Vbar)
    return o[0], lse[0]


def append_tokens(Kc, Vc, Kbar, Vbar, positions, k_new, v_new, L: int):
    """Reference semantics of appending one token per sequence, in place on
    float64 arrays: row positions[b] of every KV head takes k_new[b] and
    v_new[b]; a sequence whose append completes block blk = (pos+1)/L - 1
    gets that block's landmark recomputed as the mean of its L rows.
    Positions outside [0, C) leave the sequence unchanged."""
    B, Hkv, C, d = Kc.shape
    for b in range(B):
        pos = int(positions[b])
        if pos < 0 or pos >= C:
            continue
        Kc[b, :, pos] = k_new[b]
        Vc[b, :, pos] = v_new[b]
        if (pos + 1) % L == 0 and (pos + 1) // L <= Kbar.shape[2]:
            blk = (pos + 1) // L - 1
            Kbar[b, :, blk] = Kc[b, :, blk * L:(blk + 1) * L].mean(axis=1)
            Vbar[b, :, blk] = Vc[b, :, blk * L:(blk + 1) * L].mean(axis=1)


# ---------------------------------------------------------------------------
# Step 8: backward -- gradients of O with respect to Q, K and V for a given
# upstream gradient dO.  The pages train at these lengths ("Training at 1M+
# Token Context ...", Flash Attention and Block-Sparse Flash Attention
# paragraphs; "Million Token Context Window Optimization ...", section
# "Distributed training"), without writing the backward out; what follows is
# the chain rule applied to the forward above, nothing more:
#   P = softmax over the visible entries,  O = P V_vis
#   dP = dO V_vis^T,  D = rowsum(dO * O),  dS = P * (dP - D)
#   dQ = scale dS K_vis,  dK_vis = scale dS^T Q,  dV_vis = P^T dO
# summed over the query heads that share a KV head.  A landmark is the mean
# of its block, so each of the block's L rows receives 1/L of the
# landmark's gradient.
# ---------------------------------------------------------------------------

def _probs(S_win, M_win, S_lm, M_lm):
    """Normalised probabilities of one softmax over the visible window and
    landmark scores: (P_win, P_lm, LSE)."""
    S_win = np.where(M_win, S_win, NEG_INF)
    S_lm = np.where(M_lm, S_lm, NEG_INF)
    m = np.maximum(S_win.max(axis=1, initial=NEG_INF), S_lm.max(axis=1, initial=NEG_INF))
    P_win = np.where(M_win, np.exp(S_win - m[:, None]), 0.0)
    P_lm = np.where(M_lm, np.exp(S_lm - m[:, None]), 0.0)
    l = P_win.sum(axis=1) + P_lm.sum(axis=1)
    return P_win / l[:, None], P_lm / l[:, None], m + np.log(l)


def _softmax_bwd(P, dP, D):
    """Gradient of the scores of one softmax row: P * (dP - D)."""
    return P * (dP - D[:, None])


def _mean_bwd(dXbar, L: int):
    """Adjoint of block-mean pooling: [..., G, d] -> [..., G*L, d], every row
    of block b gets dXbar[b] / L."""
    return np.repeat(dXbar, L, axis=-2) / L


def attn_bwd(Q, K, V, dO, w: int, G: int, scale: Optional[float] = None,
             kv_heads: Optional[Sequence[int]] = None, group_span: int = 512, O=None):
    """Gradients (dQ [B, Hq, n, d], dK, dV [B, Hkv, n, d]) of the forward
    above, fp64, with landmarks the means of K and V.  ``kv_heads`` limits the
    work to those KV heads and their query heads (the other entries are
    zero).  Rows are processed in groups of nearby rows whose key range
    strictly contains their windows, as in attn().

    ``O`` is the forward output the backward is handed (as a training step
    saves it, e.g. rounded to bf16); it enters only through the softmax
    term D_i = dO_i . O_i.  By default the exact forward output is used."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    B, Hq, n, d = Q.shape
    Hkv = K.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    L = block_len(n, G) if G else 0
    Kbar = pool(K, G) if G else np.zeros((B, Hkv, 0, d))
    Vbar = pool(V, G) if G else np.zeros((B, Hkv, 0, d))
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    dKbar = np.zeros_like(Kbar)
    dVbar = np.zeros_like(Vbar)
    gsel = set(range(Hkv) if kv_heads is None else kv_heads)
    for h in range(Hq):
        g = kv_head(h, Hq, Hkv)
        if g not in gsel:
            continue
        for grp_rows in _row_groups(np.arange(n), group_span):
            lo = max(0, int(grp_rows[0]) - w)
            hi = min(n, int(grp_rows[-1]) + 2)
            M_win = window_visible(grp_rows[:, None], np.arange(lo, hi)[None, :], w)
            M_lm = (landmark_visible(grp_rows[:, None], np.arange(G)[None, :], L, w) if G
                    else np.zeros((len(grp_rows), 0), dtype=bool))
            for b in range(B):
                q = Q[b, h, grp_rows]
                do = dO[b, h, grp_rows]
                ks, vs = K[b, g, lo:hi], V[b, g, lo:hi]
                kb, vb = Kbar[b, g], Vbar[b, g]
                P_win, P_lm, _ = _probs(scale * (q @ ks.T), M_win, scale * (q @ kb.T), M_lm)
                Or = P_win @ vs + P_lm @ vb if O is None else np.asarray(O[b, h, grp_rows], np.float64)
                D = (do * Or).sum(axis=1)
                dS_win = _softmax_bwd(P_win, do @ vs.T, D)
                dS_lm = _softmax_bwd(P_lm, do @ vb.T, D)
                dQ[b, h, grp_rows] = scale * (dS_win @ ks + dS_lm @ kb)
                dK[b, g, lo:hi] += scale * (dS_win.T @ q)
                dV[b, g, lo:hi] += P_win.T @ do
                dKbar[b, g] += scale * (dS_lm.T @ q)
                dVbar[b, g] += P_lm.T @ do
    if G:
        dK += _mean_bwd(dKbar, L)
        dV += _mean_bwd(dVbar, L)
    return dQ, dK, dV


def attn_bwd_dq_rows(Q, K, V, dO, w: int, G: int, scale: Optional[float] = None,
                     rows: Optional[Dict[int, np.ndarray]] = None, group_span: int = 512, O=None):
    """dQ on selected rows only (dQ of a row needs only that row's visible
    entries): {head: (rows, dQ [B, R, d])}.  ``O``, as in attn_bwd: the
    forward output the backward is handed, {head: [B, R, d]} on the same
    rows; by default the exact one."""
    Q = np.asarray(Q)
    B, Hq, n, d = Q.shape
    Hkv = K.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    L = block_len(n, G) if G else 0
    out = {}
    for h in sorted(rows):
        g = kv_head(h, Hq, Hkv)
        r_all = np.asarray(rows[h], dtype=np.int64)
        res = np.empty((B, len(r_all), d))
        kb_all = [pool(np.asarray(K[b, g], np.float64), G) if G else np.zeros((0, d)) for b in range(B)]
        vb_all = [pool(np.asarray(V[b, g], np.float64), G) if G else np.zeros((0, d)) for b in range(B)]
        pos = 0
        for grp_rows in _row_groups(r_all, group_span):
            lo = max(0, int(grp_rows[0]) - w)
            hi = min(n, int(grp_rows[-1]) + 2)
            M_win = window_visible(grp_rows[:, None], np.arange(lo, hi)[None, :], w)
            M_lm = (landmark_visible(grp_rows[:, None], np.arange(G)[None, :], L, w) if G
                    else np.zeros((len(grp_rows), 0), dtype=bool))
            for b in range(B):
                q = np.asarray(Q[b, h, grp_rows], np.float64)
                do = np.asarray(dO[b, h, grp_rows], np.float64)
                ks = np.asarray(K[b, g, lo:hi], np.float64)
                vs = np.asarray(V[b, g, lo:hi], np.float64)
                kb, vb = kb_all[b], vb_all[b]
                P_win, P_lm, _ = _probs(scale * (q @ ks.T), M_win, scale * (q @ kb.T), M_lm)
                if O is None:
                    Or = P_win @ vs + P_lm @ vb
                else:
                    Or = np.asarray(O[h][b, pos:pos + len(grp_rows)], np.float64)
                D = (do * Or).sum(axis=1)
                dS_win = _softmax_bwd(P_win, do @ vs.T, D)
                dS_lm = _softmax_bwd(P_lm, do @ vb.T, D)
                res[b, pos:pos + len(grp_rows)] = scale * (dS_win @ ks + dS_lm @ kb)
            pos += len(grp_rows)
        out[h] = (r_all, res)
    return out


# ---------------------------------------------------------------------------
# Step 9: attention over caller-given key blocks (block-sparse lists).  The
# pages describe block-sparse kernels driven by per-block index lists with
# counts ("Sparse Attention GPU Cluster Implementation: What Actually Works",
# section on the kernel that drives the sparse pattern; 64-token blocks) and
# patterns such as 128-token blocks each attending to 16 others ("Million
# Token Context Window Optimization: What Actually Works", indexing
# section).  Reading: query block t (rows t*bq .. t*bq+bq-1) of head h sees
# every key of the key blocks listed for it (blocks of bk keys, clipped at
# n), optionally only keys j <= i (causal), under one softmax; a listed
# block index outside [0, ceil(n/bk)) contributes nothing; a block listed
# twice is seen twice.  A row that sees nothing has O = 0, LSE = -inf.
# ---------------------------------------------------------------------------

def blocksparse_mask(n: int, counts, indices, bq: int, bk: int, causal: bool) -> np.ndarray:
    """Multiplicity of each (row, key) pair for one head: int [n, n]."""
    nkb = -(-n // bk)
    M = np.zeros((n, n), dtype=np.int64)
    for t in range(-(-n // bq)):
        r0, r1 = t * bq, min(n, (t + 1) * bq)
        for c in range(int(counts[t])):
            kb = int(indices[t][c])
            if kb < 0 or kb >= nkb:
                continue
            M[r0:r1, kb * bk:min(n, (kb + 1) * bk)] += 1
    if causal:
        M = np.tril(M)
    return M


def attn_blocksparse(Q, K, V, counts, indices, bq: int, bk: int, causal: bool, scale: Optional[float] = None):
    """O [B, Hq, n, d], LSE [B, Hq, n] for per-(batch, query head) block
    lists: counts [B, Hq, T], indices [B, Hq, T, max_blocks]."""
    Q = np.asarray(Q, dtype=np.float64)
    B, Hq, n, d = Q.shape
    Hkv = K.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    O = np.zeros((B, Hq, n, d))
    LSE = np.full((B, Hq, n), NEG_INF)
    for b in range(B):
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            M = blocksparse_mask(n, counts[b][h], indices[b][h], bq, bk, causal)
            k = np.asarray(K[b, g], np.float64)
            v = np.asarray(V[b, g], np.float64)
            S = scale * (Q[b, h] @ k.T)
            vis = M > 0
            m = np.where(vis, S, NEG_INF).max(axis=1)
            live = np.isfinite(m)
            E = np.where(vis, M * np.exp(S - np.where(live, m, 0.0)[:, None]), 0.0)
            l = E.sum(axis=1)
            O[b, h, live] = (E[live] @ v) / l[live, None]
            LSE[b, h, live] = m[live] + np.log(l[live])
    return O, LSE


def attn_blocksparse_rows(Q, K, V, counts, indices, bq: int, bk: int, causal: bool, scale: Optional[float] = None,
                          rows: Optional[Dict[int, np.ndarray]] = None):
    """Selected rows of attn_blocksparse: {head: (rows, O [B, R, d],
    LSE [B, R])}.  Each row's keys are gathered from its query block's list
    (with multiplicity) and the causal predicate applied to each."""
    Q = np.asarray(Q)
    B, Hq, n, d = Q.shape
    Hkv = K.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nkb = -(-n // bk)
    out = {}
    for h in sorted(rows):
        g = kv_head(h, Hq, Hkv)
        r_all = np.asarray(rows[h], dtype=np.int64)
        O = np.zeros((B, len(r_all), d))
        LSE = np.full((B, len(r_all)), NEG_INF)
        for b in range(B):
            for k, i in enumerate(r_all):
                t = int(i) // bq
                keys = [j for c in range(int(counts[b][h][t]))
                        for kb in [int(indices[b][h][t][c])] if 0 <= kb < nkb
                        for j in range(kb * bk, min(n, (kb + 1) * bk))]
                keys = np.array([j for j in keys if not causal or j <= i], dtype=np.int64)
                if len(keys) == 0:
                    continue
                q = np.asarray(Q[b, h, i], np.float64)
                sc = scale * (np.asarray(K[b, g, keys], np.float64) @ q)
                m = sc.max()
                p = np.exp(sc - m)
                O[b, k] = (p @ np.asarray(V[b, g, keys], np.float64)) / p.sum()
                LSE[b, k] = m + np.log(p.sum())
        out[h] = (r_all, O, LSE)
    return out



def gather_pages(pool, table, page: int):
    """Contiguous caches [B, Hkv, P*page, d] of paged ones: pool
    [num_pages, Hkv, page, d], table [B, P] (logical page -> physical page).
    Entries outside [0, num_pages) give zero rows.  (The paged layout of the
    "Sparse Attention GPU Cluster Implementation" page's FAQ mention of
    PagedAttention; decode over it is decode_varlen over these caches.)"""
    pool = np.asarray(pool, np.float64)
    table = np.asarray(table)
    B, P = table.shape
    Hkv, d = pool.shape[1], pool.shape[3]
    out = np.zeros((B, Hkv, P * page, d))
    for b in range(B):
        for lp in range(P):
            pid = int(table[b, lp])
            if 0 <= pid < pool.shape[0]:
                out[b, :, lp * page:(lp + 1) * page] = pool[pid]
    return out
