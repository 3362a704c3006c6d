// Closed forms of the window + landmark visibility rule and of the
// block-sparse tile schedule.  Compiled for both host (plan exports) and
// device (kernels), so the schedule the library reports is the one it runs.
//
// Rule (page "Scaling GPU Cluster for Million Token Context", section "Why
// Sparse Attention Changes the Game", made precise): row i sees keys
// i-w < j <= i and landmark b iff (b+1)*L - 1 <= i - w, L = n / G.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

// Tile shapes.  The bf16 kernel: 128 query rows (4 wavefronts x 32 rows) by
// 64 keys.  The float32 kernel: 64 query rows by 64 keys.
constexpr int kBM_BF16 = 128;
constexpr int kBN_BF16 = 64;
constexpr int kBM_F32 = 64;
constexpr int kBN_F32 = 64;

// Lowest window key of row i.
__host__ __device__ inline int win_lo(int i, int w) {
  const int lo = i - w + 1;
  return lo > 0 ? lo : 0;
}

// Visible landmarks of row i: blocks b with (b+1)*L <= i - w + 1, i.e. the
// prefix 0 .. floor((i-w+1)/L)-1, capped at G.  The test on t avoids C's
// truncating division of negatives.
__host__ __device__ inline int lm_count(int i, int w, int G, int L) {
  if (G <= 0) return 0;
  const int t = i - w + 1;
  if (t < L) return 0;
  const int c = t / L;
  return c < G ? c : G;
}

// Work of one query tile: rows [r0, r1] (r1 already clipped to n-1).
struct TileRange {
  int r0, r1;
  int n_lm_tiles;       // landmark tiles 0 .. n_lm_tiles-1
  int lm_lo, lm_hi;     // lm_count(r0), lm_count(r1)
  int kt_lo, kt_hi;     // window key tiles kt_lo .. kt_hi (inclusive)
};

__host__ __device__ inline TileRange tile_range(int t, int BM, int BN, int n, int w, int G, int L) {
  TileRange r;
  r.r0 = t * BM;
  r.r1 = r.r0 + BM - 1 < n - 1 ? r.r0 + BM - 1 : n - 1;
  r.lm_lo = lm_count(r.r0, w, G, L);
  r.lm_hi = lm_count(r.r1, w, G, L);
  r.n_lm_tiles = (r.lm_hi + BN - 1) / BN;
  r.kt_lo = win_lo(r.r0, w) / BN;
  r.kt_hi = r.r1 / BN;
  return r;
}

// No mask needed on landmark tile lt: every row of the tile sees all of it.
__host__ __device__ inline bool lm_tile_interior(int lt, int BN, int lm_lo_rows) {
  return (lt + 1) * BN <= lm_lo_rows;
}

// No mask needed on window tile kt for rows [r0, r1]: all its keys are at or
// before r0 and after r1 - w.
__host__ __device__ inline bool win_tile_interior(int kt, int BN, int r0, int r1, int w) {
  const int k0 = kt * BN;
  return k0 + BN - 1 <= r0 && k0 >= r1 - w + 1;
}

// Decode: entries of row ctx-1 and the chunking of its ordered list.
struct DecodePlan {
  int lm;       // visible landmarks
  int win;      // window keys
  int win0;     // first window key position
  int entries;  // lm + win
  int chunk;    // entries per chunk, ceil(entries / S)
};

// Row n-1 of a sequence of n >= 0 tokens whose landmark blocks have length
// L (G blocks of capacity).  n = 0 gives an empty list (chunk 0).
__host__ __device__ inline DecodePlan decode_plan_fixed(int n, int w, int G, int L, int S) {
  DecodePlan p;
  if (n <= 0) {
    p.lm = p.win = p.win0 = p.entries = p.chunk = 0;
    return p;
  }
  const int i = n - 1;
  p.lm = lm_count(i, w, G, L);
  p.win0 = win_lo(i, w);
  p.win = i - p.win0 + 1;
  p.entries = p.lm + p.win;
  p.chunk = (p.entries + S - 1) / S;
  return p;
}

// Static decode: the whole cache of ctx tokens, L = ctx / G.
__host__ __device__ inline DecodePlan decode_plan(int ctx, int w, int G, int S) {
  return decode_plan_fixed(ctx, w, G, G > 0 ? ctx / G : 1, S);
}

}  // namespace msa
