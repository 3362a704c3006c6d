// Decode: one new query per sequence at position ctx-1 attends to its causal
// window of the KV cache plus the visible landmarks, split into chunks whose
// softmax statistics are merged afterwards (the single-GPU form of the
// Ring Attention aggregation on the page "Training at 1M+ Token Context:
// Ring Attention, YaRN, NTK-Aware Scaling GPU Cost", Ring Attention
// paragraph: partial results per KV block, combined through their softmax
// statistics, no score matrix kept).
//
// The unit of work is a wavefront streaming a range of the ordered visible
// list (landmarks, then window keys) through a private ring of LDS tiles.
// Tiles go HBM -> LDS with global loads that write LDS (addresses per lane,
// so a tile may straddle the landmark/window boundary), one tile ahead of
// the one being consumed; no registers hold in-flight data and the waves
// never wait for each other while streaming.  The query heads of the KV
// group (<= 16) form the N dimension of v_mfma_f32_16x16x32_bf16, so every
// K/V row is read once for all of them: S^T = K q^T per 16-entry block (K
// operands read row-per-lane from a row-swizzled tile), online softmax per
// head, O^T += V^T P^T with V^T read by ds_read_b64_tr_b16 from the
// row-major V tile.
//
// Two schedules, the same arithmetic up to float32 rounding of the merge:
//  * fused (many sequence x KV-head pairs): one workgroup of 4 wavefronts
//    per (sequence, KV head); wavefront w streams the consecutive chunks
//    [w*S/4, (w+1)*S/4) as one continuous tile stream and folds each
//    finished chunk's partial into a running total by its softmax
//    statistics; the 4 totals are merged through LDS and the final O and
//    LSE written by the same kernel.  Partials stay on chip (the workspace
//    is not written).
//  * split (few pairs, where chunks are the parallelism): one wavefront per
//    (sequence, KV head, chunk) writes its partial; decode_merge_kernel
//    then merges the chunks of each (sequence, query head).
#include <atomic>
#include <mutex>

#include "msa_device.hpp"
#include "msa_internal.hpp"
#include "msa_plan.hpp"

namespace msa {
namespace {


constexpr int kSplitTE = 32;  // entries per tile, split schedule
constexpr int kFusedTE = 16;  // entries per tile, fused schedule
constexpr int kFusedWaves = 4;

__device__ __forceinline__ float max16(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float sum16(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

// Wait until every vector-memory operation of this wavefront is done,
// other counters unconstrained.
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// One ring slot: K tile then V tile, TE rows of D bf16 each, 16-byte chunks
// swizzled by row: K by row mod CH (the 16 rows a K operand reads at once
// fall in distinct banks), V by 4*(row mod 4) (the 4 rows x 4 chunks a
// transpose read touches).
template <int D, int TE>
struct Tile {
  static constexpr int RB = D * 2;
  static constexpr int CH = RB / 16;
  static constexpr int BYTES = TE * RB;   // one tensor
  static constexpr int SLOT = 2 * BYTES;  // K + V
  static constexpr int KI = BYTES / 1024; // load instructions per tensor (64 lanes x 16 B)
  static constexpr int RING = 2 * SLOT;   // double buffer
  __device__ static constexpr int kswz(int r) { return r % CH; }
  __device__ static constexpr int vswz(int r) { return (r % 4) * (CH / 4); }
};

// Staging of one tile of entries e0 .. e0+cnt-1 (cnt >= 1): instruction i
// writes slot bytes i*1024 + 16*lane, i.e. tile row r = (i*64 + lane) / CH,
// LDS chunk position p = (i*64 + lane) % CH, which holds source chunk
// p ^ swizzle(r).  Entry e is landmark e if e < lm, else cache row
// win0 + e - lm; rows past cnt repeat entry e0 (finite data that gets zero
// weight).  (A device function rather than a lambda in the kernel: with the
// load builtin inside a lambda the host pass drops the kernel's launch stub.)
// Paged caches: the physical pages that this lane's rows of one tile lie
// in (at most two, logical pages lpA <= lpA + 1, since a tile spans at most
// 32 rows and pages hold at least 32), loaded one tile ahead.
struct PageIds {
  int lpA, idA, idB;
};

// With PAGED, window row r of the sequence lives at row (r mod page) of
// physical page tbl[r / page]: kc/vc are then the pools' bases for this KV
// head and pstride the bytes between consecutive physical pages of it.  A
// page id outside [0, num_pages) reads page 0 (no access leaves the pool).
template <int D, int TE>
struct Stager {
  using T = Tile<D, TE>;
  const unsigned char *kl, *vl, *kc, *vc;
  int lm, win0, lane;
  const int32_t* tbl;  // this sequence's block table (paged), else null
  int shift, max_pages, num_pages;
  size_t pstride;

  __device__ __forceinline__ int entry(int e0, int cnt, int i) const {
    const int r = (i * 64 + lane) / T::CH;
    return e0 + (r < cnt ? r : 0);
  }
  // Page ids of the tile at e0 (cnt >= 1 entries).  Its window rows are one
  // contiguous run spanning at most two pages (TE <= page), so both ids are
  // the same for every lane: they are read with uniform indices, which the
  // compiler turns into scalar loads, so the vector-memory counter that the
  // loop waits on covers only tile data.
  __device__ __forceinline__ PageIds fetch(int e0, int cnt) const {
    PageIds pg{0, 0, 0};
    const int ea = max(e0, lm);
    const int eb = e0 + cnt - 1;
    if (eb < ea) return pg;  // landmark entries only
    pg.lpA = __builtin_amdgcn_readfirstlane((win0 + ea - lm) >> shift);
    const int lpB = __builtin_amdgcn_readfirstlane((win0 + eb - lm) >> shift);
    pg.idA = tbl[__builtin_amdgcn_readfirstlane(min(pg.lpA, max_pages - 1))];
    pg.idB = tbl[__builtin_amdgcn_readfirstlane(min(lpB, max_pages - 1))];
    return pg;
  }
  template <bool PAGED>
  __device__ __forceinline__ void issue(unsigned char* slot, int e0, int cnt, const PageIds& pg) const {
#pragma unroll
    for (int i = 0; i < T::KI; ++i) {
      const int sl = i * 64 + lane;
      const int r = sl / T::CH, p = sl % T::CH;
      const int e = entry(e0, cnt, i);
      const bool is_lm = e < lm;
      // both candidate addresses, then a select (no divergent branches)
      const int row = max(win0 + e - lm, 0);
      size_t off;
      if constexpr (PAGED) {
        int id = (row >> shift) == pg.lpA ? pg.idA : pg.idB;
        id = (unsigned)id < (unsigned)num_pages ? id : 0;
        off = (size_t)id * pstride + (size_t)(row & ((1 << shift) - 1)) * T::RB;
      } else {
        off = (size_t)row * T::RB;
      }
      const size_t loff = (size_t)e * T::RB;
      const unsigned char* ks = is_lm ? kl + loff : kc + off;
      const unsigned char* vs = is_lm ? vl + loff : vc + off;
      __builtin_amdgcn_global_load_lds(ks + (p ^ T::kswz(r)) * 16, (lds_void_ptr)(slot + i * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vs + (p ^ T::vswz(r)) * 16, (lds_void_ptr)(slot + T::BYTES + i * 1024), 16,
                                       0, 0);
    }
  }
};

// Per-wavefront constants: LDS operand offsets inside a slot and the query
// fragments of the KV group's heads.
template <int D, int TE>
struct WaveOps {
  using T = Tile<D, TE>;
  static constexpr int KK = D / 32;  // k-steps of S^T = K q^T
  static constexpr int MB = D / 16;  // 16-dim blocks of O^T
  static constexpr int NBLK = TE / 16;
  static_assert(NBLK == 1 || NBLK == 2, "TE is 16 or 32");
  uint32_t kfo[NBLK][KK];  // K operand of block blk, step kk: entry blk*16 + c16, dims kk*32 + g4*8 .. +7
  uint32_t vfo[MB];        // V^T operand of block 0, dim block mb (block 1: + 16 rows)
  bf16x8 qf[KK];           // B[k = dim][n = head in group]

  __device__ __forceinline__ void init(const uint16_t* q_group, int grp, int c16, int g4) {
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) {
      const int r = blk * 16 + c16;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) kfo[blk][kk] = (uint32_t)(r * T::RB + (((kk * 4 + g4) ^ T::kswz(r)) * 16));
    }
    // transpose read: lane j of 16-lane group g4 points at entry g4*4 + j/4,
    // dims mb*16 + 4*(j%4); it receives entries g4*4 + 0..3 of dim mb*16 + j.
    // 16 rows down keeps the V swizzle (it depends on row mod 4).
    const int r = g4 * 4 + (c16 >> 2);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int d = mb * 16 + 4 * (c16 & 3);
      vfo[mb] = (uint32_t)(T::BYTES + r * T::RB + (((d / 8) ^ T::vswz(r)) * 16) + (d % 8) * 2);
    }
    const uint16_t* qp = q_group + (size_t)(c16 < grp ? c16 : 0) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (c16 < grp) v = *reinterpret_cast<const u32x4*>(qp + kk * 32 + g4 * 8);
      qf[kk] = __builtin_bit_cast(bf16x8, v);
    }
  }
};

// Online-softmax state of one wavefront for the 16 head columns: lane
// (c16, g4) holds O^T[dim mb*16 + g4*4 + i][head c16] in o[mb][i]; m is the
// running max of head c16 (log2 domain); l its partial sum over this
// lane's entries (sum16 gives the head's total).
template <int D>
struct Acc {
  f32x4 o[D / 16];
  float m, l;
  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb) o[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    m = -1e30f;
    l = 0.f;
  }
};

// One tile: S^T = K q^T, mask entries >= cnt, online softmax, O^T += V^T P^T.
template <int D, int TE>
__device__ __forceinline__ void consume_tile(const unsigned char* slot, int cnt, const WaveOps<D, TE>& w, float c2,
                                             int g4, Acc<D>& a) {
  using W = WaveOps<D, TE>;
  constexpr int KK = W::KK, MB = W::MB, NBLK = W::NBLK;
  f32x4 acc[NBLK];  // acc[blk][i] = entry blk*16 + g4*4 + i, head c16
#pragma unroll
  for (int blk = 0; blk < NBLK; ++blk) {
    acc[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(slot + w.kfo[blk][kk]);
      acc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, w.qf[kk], acc[blk], 0, 0, 0);
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int blk = 0; blk < NBLK; ++blk) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float sc = blk * 16 + g4 * 4 + i < cnt ? acc[blk][i] * c2 : -INFINITY;
      acc[blk][i] = sc;
      mx = fmaxf(mx, sc);
    }
  }
  mx = max16(mx);
  const float m_new = fmaxf(a.m, mx);
  const float alpha = __builtin_amdgcn_exp2f(a.m - m_new);
  a.m = m_new;
  a.l *= alpha;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) a.o[mb] *= alpha;
  // P^T operand: slots g4*8 + 4*blk + i <-> entry blk*16 + g4*4 + i
  uint32_t pw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int blk = 0; blk < NBLK; ++blk) {
    const float p0 = __builtin_amdgcn_exp2f(acc[blk][0] - m_new), p1 = __builtin_amdgcn_exp2f(acc[blk][1] - m_new);
    const float p2 = __builtin_amdgcn_exp2f(acc[blk][2] - m_new), p3 = __builtin_amdgcn_exp2f(acc[blk][3] - m_new);
    a.l += (p0 + p1) + (p2 + p3);
    pw[2 * blk] = pack_bf16x2(p0, p1);
    pw[2 * blk + 1] = pack_bf16x2(p2, p3);
  }
  const bf16x8 pf = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
  const uint32_t base = lds_addr(slot);
  u32x2 v[NBLK][MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) v[blk][mb] = ds_read_tr16_b64<0>(base + w.vfo[mb] + blk * 16 * Tile<D, TE>::RB);
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    if constexpr (NBLK == 2) {
      lds_wait(NBLK * (MB - 1 - mb), v[0][mb], v[1][mb]);
    } else {
      lds_wait(NBLK * (MB - 1 - mb), v[0][mb]);
    }
    // block 1 (if any) fills slots 4..7; with one block they repeat block 0 under zero weight
    const u32x2 lo = v[0][mb];
    const u32x2 hi = v[NBLK - 1][mb];
    const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
    a.o[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, a.o[mb], 0, 0, 0);
  }
}

// A chunk's partial: normalised O and natural-log LSE of heads c16 < grp
// (l already summed over the wavefront).  An empty chunk gives O = 0,
// LSE = -inf.
template <int D>
__device__ __forceinline__ void store_partial(const Acc<D>& a, float* __restrict__ ws_o, float* __restrict__ ws_lse,
                                              size_t slot0, int grp, int c16, int g4) {
  if (c16 >= grp) return;
  const size_t slot = slot0 + c16;
  const float inv = a.l > 0.f ? 1.0f / a.l : 0.f;
#pragma unroll
  for (int mb = 0; mb < D / 16; ++mb) {
    *reinterpret_cast<f32x4*>(ws_o + slot * D + mb * 16 + g4 * 4) = a.o[mb] * inv;
  }
  if (g4 == 0) ws_lse[slot] = a.l > 0.f ? (a.m + log2f(a.l)) * kLn2 : -INFINITY;
}

// Chunk c of the visible list covers entries [c*chunk, min(E, (c+1)*chunk)).
template <int TE>
struct ChunkTiles {
  int chunk, E;
  __device__ __forceinline__ int lo(int c) const { return c * chunk; }
  __device__ __forceinline__ int hi(int c) const { return min(E, (c + 1) * chunk); }
  __device__ __forceinline__ int ntile(int c) const { return (hi(c) - lo(c) + TE - 1) / TE; }
};

// Next tile to load of a wavefront that streams chunks [c, cend) tile by
// tile into a two-slot ring.
// With PAGED, pg holds the page ids of the tile about to be issued; after
// issuing, the ids of the following tile are fetched into it (they land with
// that tile's predecessor, before the wait that precedes its issue).
struct IssueCursor {
  int c, t, n_issued;
  template <bool PAGED, int D, int TE>
  __device__ __forceinline__ void next(const Stager<D, TE>& sg, const ChunkTiles<TE>& ct, unsigned char* ring,
                                       int cend, PageIds& pg) {
    if (c >= cend) return;
    const int e0 = ct.lo(c) + t * TE;
    sg.template issue<PAGED>(ring + (n_issued & 1) * Tile<D, TE>::SLOT, e0, min(TE, ct.hi(c) - e0), pg);
    ++n_issued;
    if (++t == ct.ntile(c)) {
      ++c;
      t = 0;
    }
    if constexpr (PAGED) {
      if (c < cend) {
        const int e1 = ct.lo(c) + t * TE;
        pg = sg.fetch(e1, min(TE, ct.hi(c) - e1));
      }
    }
  }
  // Page ids of the cursor's current tile (the first one to issue).
  template <bool PAGED, int D, int TE>
  __device__ __forceinline__ PageIds first(const Stager<D, TE>& sg, const ChunkTiles<TE>& ct, int cend) const {
    PageIds pg{0, 0, 0};
    if constexpr (PAGED) {
      if (c < cend) {
        const int e0 = ct.lo(c) + t * TE;
        pg = sg.fetch(e0, min(TE, ct.hi(c) - e0));
      }
    }
    return pg;
  }
};

struct DecodeArgs {
  const uint16_t *q, *Kc, *Vc, *Kb, *Vb;
  float *ws_o, *ws_lse;
  void* Out;
  float* LSE;
  int B, Hq, Hkv, ctx, G;  // ctx: cache rows per (sequence, KV head); G: landmark slots
  float c2;                // scale * log2(e)
  int lm, win0, E, chunk, S;  // plan of row ctx-1 (used when lens is null)
  const int32_t* lens;     // per-sequence lengths, or null: every sequence holds ctx tokens
  int w, L;                // window and landmark block length (lens path)
  const int32_t* table;    // paged caches: block table [B][max_pages], else null
  int page_shift, max_pages, num_pages;
};

// Plan of sequence b: the static one, or that of its own length (clamped to
// [0, ctx]; 0 gives an empty list).
__device__ __forceinline__ DecodePlan seq_plan(const DecodeArgs& A, int b) {
  if (A.lens == nullptr) {
    DecodePlan p;
    p.lm = A.lm;
    p.win0 = A.win0;
    p.entries = A.E;
    p.chunk = A.chunk;
    p.win = A.E - A.lm;
    return p;
  }
  int n = A.lens[b];
  n = n < 0 ? 0 : (n > A.ctx ? A.ctx : n);
  return decode_plan_fixed(n, A.w, A.G, A.L, A.S);
}

template <bool PAGED, int D, int TE>
__device__ __forceinline__ Stager<D, TE> make_stager(const DecodeArgs& A, int bk, int lane, const DecodePlan& p) {
  const unsigned char* kc;
  const unsigned char* vc;
  const int32_t* tbl = nullptr;
  size_t pstride = 0;
  if constexpr (PAGED) {
    // pools [num_pages][Hkv][page][D]: this KV head's rows of page id start
    // at (id * Hkv + kvh) * page * D
    const int kvh = bk % A.Hkv, b = bk / A.Hkv;
    const size_t page_elems = (size_t)D << A.page_shift;
    kc = reinterpret_cast<const unsigned char*>(A.Kc + (size_t)kvh * page_elems);
    vc = reinterpret_cast<const unsigned char*>(A.Vc + (size_t)kvh * page_elems);
    pstride = (size_t)A.Hkv * page_elems * 2;
    tbl = A.table + (size_t)b * A.max_pages;
  } else {
    kc = reinterpret_cast<const unsigned char*>(A.Kc + (size_t)bk * A.ctx * D);
    vc = reinterpret_cast<const unsigned char*>(A.Vc + (size_t)bk * A.ctx * D);
  }
  const unsigned char* kl = kc;
  const unsigned char* vl = vc;
  if (A.G > 0) {
    kl = reinterpret_cast<const unsigned char*>(A.Kb + (size_t)bk * A.G * D);
    vl = reinterpret_cast<const unsigned char*>(A.Vb + (size_t)bk * A.G * D);
  }
  return Stager<D, TE>{kl, vl, kc, vc, p.lm, p.win0, lane, tbl, A.page_shift, A.max_pages, A.num_pages, pstride};
}

// ---------------------------------------------------------------------------
// Split schedule, pass 1: one wavefront per (sequence, KV head, chunk).
template <int D, int TE, bool PAGED>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeArgs A) {
  using T = Tile<D, TE>;
  __shared__ __align__(16) unsigned char ring[T::RING];
  const int c = blockIdx.x % A.S;
  const int bk = blockIdx.x / A.S;  // b * Hkv + kvh
  const int b = bk / A.Hkv, kvh = bk % A.Hkv;
  const int grp = A.Hq / A.Hkv;
  const int lane = threadIdx.x, c16 = lane & 15, g4 = lane >> 4;

  const DecodePlan p = seq_plan(A, b);
  const int e_beg = c * p.chunk;
  const int e_end = min(p.entries, e_beg + p.chunk);
  const int n_t = e_end > e_beg ? (e_end - e_beg + TE - 1) / TE : 0;
  const Stager<D, TE> sg = make_stager<PAGED, D, TE>(A, bk, lane, p);
  WaveOps<D, TE> w;
  w.init(A.q + ((size_t)b * A.Hq + kvh * grp) * D, grp, c16, g4);
  Acc<D> a;
  a.reset();

  // with PAGED, pg holds the page ids of the next tile to issue
  PageIds pg{0, 0, 0};
  if constexpr (PAGED) {
    if (n_t > 0) pg = sg.fetch(e_beg, min(TE, e_end - e_beg));
  }
  if (n_t > 0) sg.template issue<PAGED>(ring, e_beg, min(TE, e_end - e_beg), pg);
  if constexpr (PAGED) {
    if (n_t > 1) pg = sg.fetch(e_beg + TE, min(TE, e_end - e_beg - TE));
  }
  for (int t = 0; t < n_t; ++t) {
    wait_vmcnt0();  // tile t is in LDS (and tile t+1's page ids loaded); tile t-1's slot was consumed
    if (t + 1 < n_t) {
      const int e1 = e_beg + (t + 1) * TE;
      sg.template issue<PAGED>(ring + ((t + 1) & 1) * T::SLOT, e1, min(TE, e_end - e1), pg);
      if constexpr (PAGED) {
        const int e2 = e1 + TE;
        if (t + 2 < n_t) pg = sg.fetch(e2, min(TE, e_end - e2));
      }
    }
    const int e0 = e_beg + t * TE;
    consume_tile<D, TE>(ring + (t & 1) * T::SLOT, min(TE, e_end - e0), w, A.c2, g4, a);
  }
  a.l = sum16(a.l);
  store_partial<D>(a, A.ws_o, A.ws_lse, ((size_t)c * A.B + b) * A.Hq + kvh * grp, grp, c16, g4);
}

// ---------------------------------------------------------------------------
// Fused schedule: one workgroup of kFusedWaves wavefronts per (sequence,
// KV head); chunk partials, their merge and the final output in one pass.
template <int D, int TE, bool OUT_BF16, bool PAGED>
__global__ __launch_bounds__(64 * kFusedWaves) void decode_fused_kernel(DecodeArgs A) {
  // (A.ws_o, A.ws_lse unused)
  using T = Tile<D, TE>;
  constexpr int MB = D / 16;
  __shared__ __align__(16) unsigned char smem[kFusedWaves * T::RING];
  static_assert((2 * 16 + 16 * D) * 4 <= T::RING, "merge record fits a ring");
  const int bk = blockIdx.x;
  const int b = bk / A.Hkv, kvh = bk % A.Hkv;
  const int grp = A.Hq / A.Hkv;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63, c16 = lane & 15, g4 = lane >> 4;
  unsigned char* ring = smem + wave * T::RING;

  // chunks of this wavefront; chunk c is non-empty iff c * chunk < E
  const DecodePlan p = seq_plan(A, b);
  const int c0 = wave * A.S / kFusedWaves;
  const int c1 = (wave + 1) * A.S / kFusedWaves;
  const int n_ne = p.chunk > 0 ? (p.entries + p.chunk - 1) / p.chunk : 0;
  const int cend = min(c1, n_ne);
  const ChunkTiles<TE> ct{p.chunk, p.entries};

  const Stager<D, TE> sg = make_stager<PAGED, D, TE>(A, bk, lane, p);
  WaveOps<D, TE> w;
  w.init(A.q + ((size_t)b * A.Hq + kvh * grp) * D, grp, c16, g4);

  // issue cursor over the wavefront's tiles, chunk by chunk
  IssueCursor cursor{c0, 0, 0};
  Acc<D> tot, cur;
  tot.reset();
  cur.reset();
  int n_used = 0;
  PageIds pg = cursor.first<PAGED, D, TE>(sg, ct, cend);
  cursor.next<PAGED, D, TE>(sg, ct, ring, cend, pg);
  for (int c = c0; c < cend; ++c) {
    const int nt = ct.ntile(c);
    for (int t = 0; t < nt; ++t) {
      wait_vmcnt0();  // this tile is in LDS (and the next tile's page ids); the other slot was consumed
      cursor.next<PAGED, D, TE>(sg, ct, ring, cend, pg);
      const int e0 = ct.lo(c) + t * TE;
      consume_tile<D, TE>(ring + (n_used & 1) * T::SLOT, min(TE, ct.hi(c) - e0), w, A.c2, g4, cur);
      ++n_used;
    }
    // Fold the finished chunk into the wavefront's total.  Its partial is
    // not written out: a store here would make the next tile's wait (which
    // counts stores too) stall on the store's completion.
    cur.l = sum16(cur.l);
    const float mt = fmaxf(tot.m, cur.m);
    const float at = __builtin_amdgcn_exp2f(tot.m - mt), ac = __builtin_amdgcn_exp2f(cur.m - mt);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) tot.o[mb] = tot.o[mb] * at + cur.o[mb] * ac;
    tot.l = tot.l * at + cur.l * ac;
    tot.m = mt;
    cur.reset();
  }
  // merge the wavefronts' totals: waves 1.. publish (m, l, O) in their own
  // ring (no tile is in flight any more), wave 0 combines and writes.
  float* rec = reinterpret_cast<float*>(ring);  // m[16], l[16], o[16][D]
  if (wave != 0) {
    if (g4 == 0) {
      rec[c16] = tot.m;
      rec[16 + c16] = tot.l;
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) *reinterpret_cast<f32x4*>(rec + 32 + c16 * D + mb * 16 + g4 * 4) = tot.o[mb];
  }
  __syncthreads();
  if (wave != 0 || c16 >= grp) return;
  float M = tot.m;
#pragma unroll
  for (int v = 1; v < kFusedWaves; ++v) M = fmaxf(M, reinterpret_cast<const float*>(smem + v * T::RING)[c16]);
  const float a0 = __builtin_amdgcn_exp2f(tot.m - M);
  float L = tot.l * a0;
  f32x4 o[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) o[mb] = tot.o[mb] * a0;
#pragma unroll
  for (int v = 1; v < kFusedWaves; ++v) {
    const float* r = reinterpret_cast<const float*>(smem + v * T::RING);
    const float av = __builtin_amdgcn_exp2f(r[c16] - M);
    L += r[16 + c16] * av;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) o[mb] += *reinterpret_cast<const f32x4*>(r + 32 + c16 * D + mb * 16 + g4 * 4) * av;
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  const size_t row = ((size_t)b * A.Hq + kvh * grp + c16) * D;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const f32x4 val = o[mb] * inv;
    if constexpr (OUT_BF16) {
      const u32x2 pk = {pack_bf16x2(val[0], val[1]), pack_bf16x2(val[2], val[3])};
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(A.Out) + row + mb * 16 + g4 * 4) = pk;
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(A.Out) + row + mb * 16 + g4 * 4) = val;
    }
  }
  if (A.LSE != nullptr && g4 == 0) A.LSE[(size_t)b * A.Hq + kvh * grp + c16] = (M + log2f(L)) * kLn2;
}

// One wavefront per (sequence, query head): every chunk's LSE is loaded at
// once (lane c holds chunk c), the weights are reduced in-wave, then the
// chunk outputs are streamed with their loads issued ahead.
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(256) void decode_merge_kernel(const float* __restrict__ ws_o,
                                                           const float* __restrict__ ws_lse,
                                                           void* __restrict__ Out, float* __restrict__ LSE,
                                                           int BH, int S) {
  constexpr int kPer = D / 64;
  const int bh = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (bh >= BH) return;
  float M = -INFINITY;
  for (int c = lane; c < S; c += 64) M = fmaxf(M, ws_lse[(size_t)c * BH + bh]);
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) M = fmaxf(M, __shfl_xor(M, sh));
  float acc[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) acc[e] = 0.f;
  float tot = 0.f;
  for (int c0 = 0; c0 < S; c0 += 64) {
    const int c = c0 + lane;
    const float lc = c < S ? ws_lse[(size_t)c * BH + bh] : -INFINITY;
    const float wl = lc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((lc - M) * kLog2e);  // empty chunk: 0
    tot += wl;
    const int nc = min(64, S - c0);
    constexpr int kU = 32;
    for (int cc = 0; cc < nc; cc += kU) {
      float v[kU][kPer];
      float wt[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int ci = min(cc + u, nc - 1);
        wt[u] = cc + u < nc ? __shfl(wl, ci) : 0.f;
        const float* oc = ws_o + ((size_t)(c0 + ci) * BH + bh) * D;
#pragma unroll
        for (int e = 0; e < kPer; ++e) v[u][e] = oc[lane + 64 * e];
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
#pragma unroll
        for (int e = 0; e < kPer; ++e) acc[e] = fmaf(wt[u], v[u][e], acc[e]);
      }
    }
  }
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) tot += __shfl_xor(tot, sh);
  const float inv = tot > 0.f ? 1.0f / tot : 0.f;  // every chunk empty: O = 0, LSE = -inf
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const float val = acc[e] * inv;
    if constexpr (OUT_BF16) {
      static_cast<uint16_t*>(Out)[(size_t)bh * D + lane + 64 * e] = f32_to_bf16_bits(val);
    } else {
      static_cast<float*>(Out)[(size_t)bh * D + lane + 64 * e] = val;
    }
  }
  if (LSE != nullptr && lane == 0) LSE[bh] = tot > 0.f ? M + logf(tot) : -INFINITY;
}

// Compute units of the current device, cached per device (relaxed atomics:
// concurrent first calls on several threads store the same value).
int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// The fused schedule needs enough (sequence, KV head) pairs to fill the
// chip with one workgroup each and at least one chunk per wavefront; the
// descriptor's schedule field can force either.
bool use_fused(const msa_decode_desc& d) {
  if (d.schedule == MSA_DECODE_SPLIT) return false;
  if (d.schedule == MSA_DECODE_FUSED) return true;
  return (long long)d.batch * d.heads_kv >= 2LL * device_cus() && d.num_splits >= kFusedWaves;
}

template <int D, bool PAGED>
hipError_t launch_t(const msa_decode_desc& d, const DecodeArgs& A, float* ws_o, float* ws_lse, void* O, float* LSE,
                    hipStream_t stream) {
  const long long pairs = (long long)d.batch * d.heads_kv;
  if (use_fused(d)) {
    if (d.out_dtype == MSA_DTYPE_BF16) {
      hipLaunchKernelGGL((decode_fused_kernel<D, kFusedTE, true, PAGED>), dim3((unsigned)pairs),
                         dim3(64 * kFusedWaves), 0, stream, A);
    } else {
      hipLaunchKernelGGL((decode_fused_kernel<D, kFusedTE, false, PAGED>), dim3((unsigned)pairs),
                         dim3(64 * kFusedWaves), 0, stream, A);
    }
    return hipGetLastError();
  }
  hipLaunchKernelGGL((decode_split_kernel<D, kSplitTE, PAGED>), dim3((unsigned)(pairs * d.num_splits)), dim3(64), 0,
                     stream, A);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int BH = d.batch * d.heads_q;
  const int blocks = (BH + 3) / 4;
  if (d.out_dtype == MSA_DTYPE_BF16) {
    hipLaunchKernelGGL((decode_merge_kernel<D, true>), dim3(blocks), dim3(256), 0, stream, ws_o, ws_lse, O,
                       LSE, BH, d.num_splits);
  } else {
    hipLaunchKernelGGL((decode_merge_kernel<D, false>), dim3(blocks), dim3(256), 0, stream, ws_o, ws_lse, O,
                       LSE, BH, d.num_splits);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const msa_decode_desc& d, const void* q, const void* Kc, const void* Vc,
                         const void* Kbar, const void* Vbar, const int32_t* lens, const DecodePaging* paging,
                         float* ws_o, float* ws_lse, void* O, float* LSE, hipStream_t stream) {
  const DecodePlan p = decode_plan(d.ctx_len, d.window, d.num_landmarks, d.num_splits);
  const int L = d.num_landmarks > 0 ? d.ctx_len / d.num_landmarks : 1;
  DecodeArgs A{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(Kc), static_cast<const uint16_t*>(Vc),
               static_cast<const uint16_t*>(Kbar), static_cast<const uint16_t*>(Vbar), ws_o, ws_lse, O, LSE,
               d.batch, d.heads_q, d.heads_kv, d.ctx_len, d.num_landmarks, d.scale * kLog2e, p.lm, p.win0,
               p.entries, p.chunk, d.num_splits, lens, d.window, L, nullptr, 0, 0, 0};
  if (paging != nullptr) {
    A.table = paging->table;
    A.page_shift = paging->page_shift;
    A.max_pages = paging->max_pages;
    A.num_pages = paging->num_pages;
    return d.head_dim == 128 ? launch_t<128, true>(d, A, ws_o, ws_lse, O, LSE, stream)
                             : launch_t<64, true>(d, A, ws_o, ws_lse, O, LSE, stream);
  }
  return d.head_dim == 128 ? launch_t<128, false>(d, A, ws_o, ws_lse, O, LSE, stream)
                           : launch_t<64, false>(d, A, ws_o, ws_lse, O, LSE, stream);
}

bool decode_uses_split(const msa_decode_desc& d) { return !use_fused(d); }

// Per-chunk partials of the allocation-free decode: a library-owned device
// array, one copy on every GPU the library runs on, held until the process
// ends.  Host code never passes `scratch` itself to a kernel -- on the host
// the name is only a stand-in -- but the device address that
// hipGetSymbolAddress reports for the current device.  The split kernel
// writes every (chunk, sequence, query head) slot the merge reads, so
// nothing needs clearing between calls.
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

hipError_t noalloc_scratch(float** ptr) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = static_cast<float*>(addr[dev]);
  return hipSuccess;
}

}  // namespace msa
