"""Pins of the oracle's integer artefacts -- the per-row plan (lowest
visible key, number of visible landmarks), the block-sparse tile set with
its interior flags, the decode chunk bounds and the visible-pair totals --
against facts fixed outside the oracle:

* brute force over every (row, key) slot of every tile, with the masks
  written out here from the pattern's definition (query i sees key j iff
  i - w < j <= i, and landmark b iff its block's last position (b+1)L - 1
  is at or before i - w; "Scaling GPU Cluster for Million Token Context",
  section "Why Sparse Attention Changes the Game"), over tiny ragged
  shapes where every tile can be checked;
* closed forms derived from the same definition (window pairs
  w(w+1)/2 + (n-w)w per head; a row sees min(i+1, w) keys and
  clamp(floor((i-w+1)/L), 0, G) landmarks; a query tile spans the key
  tiles from floor(max(0, r0-w+1)/BN) to floor(r1/BN));
* the per-head totals and the chunk split of the decode workload worked
  out by hand for the workloads (512K context: 508 landmarks + 4096 window
  keys = 4604 entries, 16 chunks of ceil(4604/16) = 288).

Block-sparse kernels are driven by per-block index lists ("Sparse
Attention GPU Cluster Implementation: What Actually Works", section
"Sparse Attention Kernel Placement Strategies"), so the tile set must be
exact, not merely sufficient."""
import numpy as np
import pytest

from oracle import msa_oracle as orc


# ------------------------------------------------ masks from the definition

def masks_by_definition(n, w, G):
    """[n, n] window mask and [n, G] landmark mask, one Python comparison
    per slot (independent of the oracle's predicates)."""
    L = n // G if G else 0
    win = np.zeros((n, n), dtype=bool)
    lm = np.zeros((n, G), dtype=bool)
    for i in range(n):
        for j in range(n):
            win[i, j] = (i - w < j) and (j <= i)
        for b in range(G):
            lm[i, b] = (b + 1) * L - 1 <= i - w
    return win, lm


def brute_tiles(n, w, G, BM, BN):
    """Every (query tile, key tile) pair checked slot by slot: listed iff
    any slot is visible, interior iff every slot is (key or landmark slots
    past the end count as not visible; rows past n do not exist)."""
    win, lm = masks_by_definition(n, w, G)
    T = -(-n // BM)
    KT = -(-n // BN)
    LT = -(-G // BN) if G else 0
    out = []
    for t in range(T):
        rows = range(t * BM, min(n, (t + 1) * BM))
        for lt in range(LT):
            vis = [lm[i, b] if b < G else False for i in rows for b in range(lt * BN, (lt + 1) * BN)]
            if any(vis):
                out.append((t, 0, lt, all(vis)))
        for kt in range(KT):
            vis = [win[i, j] if j < n else False for i in rows for j in range(kt * BN, (kt + 1) * BN)]
            if any(vis):
                out.append((t, 1, kt, all(vis)))
    return out


def _divisors(n):
    return [g for g in range(1, n + 1) if n % g == 0]


TILE_CASES = []
for _n in (1, 17, 64, 96, 130, 200, 257):
    for _w in sorted({1, 2, 63, 64, 65, _n, 2 * _n}):
        for _G in sorted({0, 1, _n} | set(_divisors(_n)[1:4])):
            for _bm, _bn in ((128, 64), (64, 64), (32, 16)):
                TILE_CASES.append((_n, _w, _G, _bm, _bn))


@pytest.mark.parametrize("n,w,G,BM,BN", TILE_CASES)
def test_tile_plan_equals_brute_force(n, w, G, BM, BN):
    assert orc.tile_plan(n, w, G, BM, BN) == brute_tiles(n, w, G, BM, BN)


@pytest.mark.parametrize("n,w,G", [(300, 1, 0), (300, 2, 3), (300, 63, 10), (300, 64, 300), (300, 65, 5),
                                   (300, 300, 60), (300, 600, 2), (257, 40, 257), (1, 1, 1), (5, 3, 5)])
def test_row_plan_equals_brute_force(n, w, G):
    win, lm = masks_by_definition(n, w, G)
    want_lo = np.array([min(j for j in range(n) if win[i, j]) for i in range(n)])
    want_cnt = np.array([sum(int(lm[i, b]) for b in range(G)) for i in range(n)])
    lo, cnt = orc.row_plan(n, w, G)
    np.testing.assert_array_equal(lo, want_lo)
    np.testing.assert_array_equal(cnt, want_cnt)
    # a subset of rows in any order gives the same per-row values
    rows = np.random.default_rng(n + w + G).permutation(n)[: max(1, n // 3)]
    lo_s, cnt_s = orc.row_plan(n, w, G, rows)
    np.testing.assert_array_equal(lo_s, want_lo[rows])
    np.testing.assert_array_equal(cnt_s, want_cnt[rows])


# ---------------------------------------------------------- closed forms

def row_closed_form(i, w, G, L):
    """Keys and landmarks row i sees, from the definition solved for counts."""
    keys = min(i + 1, w)
    lms = 0
    if G and i - w + 1 >= 0:
        lms = min(G, (i - w + 1) // L)
    return keys, lms


@pytest.mark.parametrize("n,w,G", [(2048, 256, 16), (4096, 100, 64), (1000, 2000, 8), (777, 1, 7),
                                   (4096, 4096, 4096), (512, 33, 0)])
def test_row_plan_matches_closed_form(n, w, G):
    L = n // G if G else 0
    lo, cnt = orc.row_plan(n, w, G)
    for i in range(n):
        keys, lms = row_closed_form(i, w, G, L)
        assert i - lo[i] + 1 == keys
        assert cnt[i] == lms


def tile_counts_closed_form(n, w, G, BM, BN):
    """(window tiles, landmark tiles) per head from the closed forms."""
    L = n // G if G else 0
    win = lm = 0
    for t in range(-(-n // BM)):
        r0, r1 = t * BM, min(n - 1, t * BM + BM - 1)
        win += r1 // BN - max(0, r0 - w + 1) // BN + 1
        if G:
            lm += -(-row_closed_form(r1, w, G, L)[1] // BN)
    return win, lm


@pytest.mark.parametrize("n,w,G", [(2048, 256, 16), (2000, 300, 8), (4096, 64, 4096), (1024, 5000, 4)])
def test_tile_plan_counts_match_closed_form(n, w, G):
    plan = orc.tile_plan(n, w, G, 128, 64)
    win = sum(1 for p in plan if p[1] == 1)
    lm = sum(1 for p in plan if p[1] == 0)
    assert (win, lm) == tile_counts_closed_form(n, w, G, 128, 64)


# Per-head totals worked out for the workloads (128-row query tiles,
# 64-key tiles).  Window pairs: w(w+1)/2 + (n-w)w.  Landmark pairs: sum
# over rows i >= w-1 of min(G, floor((i-w+1)/L)).
WORKLOAD_TOTALS = {
    # name: (n, w, G, window tiles, landmark tiles, window pairs, landmark pairs)
    "tiny_fp32": (2048, 256, 16, 90, 14, 491_648, 11_662),
    "bf16_32k": (32768, 4096, 512, 15_840, 896, 125_831_168, 6_408_640),
    "gqa_128k": (131072, 4096, 512, 66_528, 4_344, 528_484_352, 31_427_056),
}


@pytest.mark.parametrize("name", sorted(WORKLOAD_TOTALS))
def test_workload_pair_totals(name):
    n, w, G, _, _, wp, lp = WORKLOAD_TOTALS[name]
    L = n // G
    assert w * (w + 1) // 2 + (n - w) * w == wp
    t = np.arange(0, n - w + 1, dtype=np.int64)  # t = i - w + 1 over rows i >= w - 1
    assert int(np.minimum(G, t // L).sum()) == lp
    assert orc.visible_pairs(n, w, G) == (wp, lp)


@pytest.mark.parametrize("name", sorted(WORKLOAD_TOTALS))
def test_workload_tile_totals(name):
    n, w, G, wt, lt, _, _ = WORKLOAD_TOTALS[name]
    assert tile_counts_closed_form(n, w, G, 128, 64) == (wt, lt)
    plan = orc.tile_plan(n, w, G, 128, 64)
    assert (sum(1 for p in plan if p[1] == 1), sum(1 for p in plan if p[1] == 0)) == (wt, lt)


# ---------------------------------------------------------- decode chunks

def test_chunk_bounds_decode_workload():
    # 512K context, window 4096, 512 landmarks of 1024 tokens: the last row
    # sees landmarks 0..507 (block 507 ends at 520191 = 524287 - 4096, exactly
    # at i - w) and 4096 window keys; 16 chunks of ceil(4604 / 16) = 288.
    kinds, idx = orc.visible_list(524287, 524288, 4096, 512)
    assert len(idx) == 4604 and int((kinds == 0).sum()) == 508
    want = [0, 288, 576, 864, 1152, 1440, 1728, 2016, 2304, 2592, 2880, 3168, 3456, 3744, 4032, 4320, 4604]
    assert orc.chunk_bounds(4604, 16).tolist() == want


def test_chunk_bounds_with_empty_chunks():
    # 5 entries over 16 chunks: one entry each, then 11 empty chunks
    assert orc.chunk_bounds(5, 16).tolist() == [0, 1, 2, 3, 4] + [5] * 12
    # 17 entries over 16 chunks: 2 each, the ninth chunk holds the last one
    assert orc.chunk_bounds(17, 16).tolist() == [0, 2, 4, 6, 8, 10, 12, 14, 16] + [17] * 8
    assert orc.chunk_bounds(0, 4).tolist() == [0, 0, 0, 0, 0]
    assert orc.chunk_bounds(7, 1).tolist() == [0, 7]


@pytest.mark.parametrize("E,S", [(1, 1), (3, 2), (100, 7), (4604, 16), (4604, 5000), (64, 64), (65, 64)])
def test_chunk_bounds_properties(E, S):
    b = orc.chunk_bounds(E, S)
    sizes = np.diff(b)
    assert b[0] == 0 and b[-1] == E and len(b) == S + 1
    assert (sizes >= 0).all()
    # every non-empty chunk but the last non-empty one holds exactly the
    # largest size, which is the smallest that fits E entries in S chunks
    s = int(sizes.max())
    assert s * S >= E and (s - 1) * S < E
    nz = np.nonzero(sizes)[0]
    assert (sizes[nz[:-1]] == s).all() and (sizes[nz[-1] + 1:] == 0).all()
