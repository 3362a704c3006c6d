// Sparse-attention prefill for bf16 inputs on gfx950 (MI355X).
//
// What it computes: for every query row i, one softmax over the causal
// window keys i-w < j <= i and the landmarks b with (b+1)*L-1 <= i-w, with
// O and the natural-log LSE as outputs (the local-window + landmark pattern
// of "Scaling GPU Cluster for Million Token Context", sections "Why Sparse
// Attention Changes the Game" and "What is Flash-MSA Sparse Attention in GPU
// Clusters?": one fused pass, tiles kept on chip, scores never written out).
//
// How, on CDNA4:
//  * A query tile is BM = 128 rows of one head (4 wavefronts x 32 rows).
//    Its walk visits only the key tiles that matter: the landmark tiles
//    0 .. ceil(c(r_last)/64)-1, then the window tiles covering
//    [r_first-w+1, r_last] (closed forms in msa_plan.hpp).  Masks are
//    evaluated only on edge tiles.
//  * Both contractions run on v_mfma_f32_32x32x16_bf16.  Scores are formed
//    transposed, S^T = K Q^T, so each lane's accumulator holds 16 keys of
//    one query row -- the B-operand layout of O^T += V^T P^T.  P never
//    leaves registers; a row's max and sum need one lane-half swap
//    (v_permlane32_swap); the rescale of O is a per-lane scalar.
//  * Softmax in base 2 with scale*log2(e) folded into one FMA per score,
//    raw v_exp_f32, packed bf16 converts.  O is normalised by the bf16 dot2
//    sum of the packed P (exactly the P that multiplies V, so a dominant key
//    gives O = its value), LSE by a float32 sum of P.  The reference max is
//    raised only when a tile's P, summed over one lane's 32 keys, exceeds
//    2^8; until then P stays bounded by 256 and O and the sums are not
//    rescaled -- exact, since they share the same reference.  The common
//    case thus costs one compare on the float32 sum and never forms a max.
//  * K and V tiles go from HBM straight into LDS (buffer loads with the LDS
//    destination; no registers, no vector ALU work), row-major with 16-byte
//    chunks XOR-swizzled by row.  K operands are row-per-lane 16-byte reads;
//    V^T operands come from row-major V through the CDNA4 transpose read
//    ds_read_b64_tr_b16.  Both swizzles make those reads conflict-free.
//    The buffer range check skips rows past the end; those LDS rows keep
//    finite earlier contents and are masked.
//  * A workgroup is 4 wavefronts with double-buffered K/V tiles and one
//    barrier per tile; two workgroups share a CU, so each SIMD runs two
//    wavefronts whose matrix-core and vector-ALU work interleave.
//  * Workgroups are renumbered XCD-aware: each XCD sweeps one KV head's
//    query tiles from the last (heaviest) to the first, all query heads of
//    the group back to back, so K/V tiles are shared in that XCD's L2.
#include "msa_device.hpp"
#include "msa_internal.hpp"
#include "msa_plan.hpp"

namespace msa {
namespace {

constexpr int BM = kBM_BF16;  // 128
constexpr int BN = kBN_BF16;  // 64
constexpr int kThreads = 256;
constexpr float kMaxTileSum = 256.0f;  // bound on one lane's sum of unnormalised P over a tile

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;

// ---------------------------------------------------------------------------
// LDS tiles: 64 rows (keys) x D bf16, row-major, 16-byte chunks permuted
// within a row.  K: chunk c of row r sits at slot c ^ (r mod CH), so the 16
// rows a K-operand read touches at once land on 16 distinct slots.  V:
// chunk c of row r sits at slot c ^ ((r mod 4) * CH/4), so the 4 rows x 4
// chunks a transpose read touches land on 16 distinct slots.
template <int D>
struct Smem {
  static constexpr int RB = D * 2;      // bytes per row
  static constexpr int CH = RB / 16;    // 16-byte chunks per row
  static constexpr int TILE = BN * RB;  // bytes per tile
  static constexpr int BYTES = 4 * TILE;
  __device__ static constexpr int kbuf(int i) { return i * TILE; }
  __device__ static constexpr int vbuf(int i) { return (2 + i) * TILE; }
  __device__ static constexpr int kswz(int r) { return r % CH; }
  __device__ static constexpr int vswz(int r) { return (r % 4) * (CH / 4); }
};

// Issues the direct-to-LDS loads of one 64-key tile for the threads of a
// 256-thread group: instruction i of wavefront wv fills LDS bytes
// [i*4096 + wv*1024, +1024) of the tile, lane l the 16 bytes at l*16.
template <int D>
struct Stager {
  using SM = Smem<D>;
  static constexpr int kInsts = SM::TILE / (kThreads * 16);  // 4 (D=128), 2 (D=64)
  uint32_t koff[kInsts];  // global byte offsets within a tile, K swizzle
  uint32_t voff[kInsts];  // same, V swizzle
  int wv;

  __device__ void init(int gtid) {
    wv = wave_index(gtid);
    const int lane = gtid & 63;
#pragma unroll
    for (int i = 0; i < kInsts; ++i) {
      const int q = (i * 4 + wv) * 64 + lane;  // 16-byte slot index within the tile
      const int r = q / SM::CH;
      const int slot = q % SM::CH;
      koff[i] = (uint32_t)(r * SM::RB + ((slot ^ SM::kswz(r)) * 16));
      voff[i] = (uint32_t)(r * SM::RB + ((slot ^ SM::vswz(r)) * 16));
    }
  }
  __device__ void issue(__amdgpu_buffer_rsrc_t rsrc, const uint32_t* off, unsigned char* tile, int row0) const {
    const uint32_t soff = (uint32_t)row0 * SM::RB;
#pragma unroll
    for (int i = 0; i < kInsts; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_ptr)(tile + i * 4096 + wv * 1024), 16, off[i], soff,
                                               0, 0);
    }
  }
  __device__ void issue_k(__amdgpu_buffer_rsrc_t r, unsigned char* tile, int row0) const {
    issue(r, koff, tile, row0);
  }
  __device__ void issue_v(__amdgpu_buffer_rsrc_t r, unsigned char* tile, int row0) const {
    issue(r, voff, tile, row0);
  }
};

// Per-lane LDS offsets of the MFMA operands within a tile.
//  K operand of S^T = K Q^T, k-step ks, 32-key block mb: row mb*32 + r32,
//    dims ks*16 + g2*8 .. +7 (one 16-byte read).
//  V^T operand of O^T += V^T P^T, 16-key step kk, 32-dim block db: two
//    transpose reads of 4 keys x 4 dims per lane; within each 16-lane group
//    lane j points at key (base + j/4), dims (dbase + 4*(j%4)); the read
//    hands lane j the 4 keys of dim dbase + j.
template <int D>
struct Frag {
  using SM = Smem<D>;
  uint32_t k[D / 16];  // per ks (mb adds 32 rows)
  uint32_t v[D / 32];  // per db (kk adds 16 rows, the second read 8 rows)

  __device__ void init(int lane) {
    const int r32 = lane & 31, g2 = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const int c = ks * 2 + g2;
      k[ks] = (uint32_t)(r32 * SM::RB + ((c ^ SM::kswz(r32)) * 16));
    }
    const int g = lane >> 4, j = lane & 15;
    const int key = (g >> 1) * 4 + (j >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int d = db * 32 + (g & 1) * 16 + 4 * (j & 3);
      const int c = d / 8;
      v[db] = (uint32_t)(key * SM::RB + ((c ^ SM::vswz(key)) * 16) + (d % 8) * 2);
    }
  }
};

// ---------------------------------------------------------------------------
// Per-lane running state of one query row (shared with the lane l^32).
template <int D>
struct RowState {
  f32x16 o[D / 32];  // O^T accumulators: o[db][jj*4+i] = dim db*32 + jj*8 + g2*4 + i
  float m;           // running reference max (base-2 units)
  float l;           // this lane's share of sum(bf16 P): normalises O
  float ls;          // this lane's share of sum(P) in float32: gives LSE
};

// Which keys of a tile a wavefront's rows [wr0, wr1] see: visit the tile at
// all (any) and apply no mask (interior).
struct TileVis {
  bool any, interior;
};

__device__ __forceinline__ TileVis tile_vis(bool is_lm, int key0, int wr0, int wr1, int wlm_lo, int wlm_hi,
                                            int w) {
  TileVis v;
  if (is_lm) {
    v.any = key0 < wlm_hi;
    v.interior = key0 + BN <= wlm_lo;
  } else {
    v.any = key0 <= wr1 && key0 + BN - 1 >= wr0 - w + 1;
    v.interior = key0 + BN - 1 <= wr0 && key0 >= wr1 - w + 1;
  }
  return v;
}

// -inf on every score this lane's row does not see.
__device__ __forceinline__ void mask_tile(f32x16* s, bool is_lm, int key0, int row, int lmc, int w, int g2) {
  const int base = row - key0 - g2 * 4;  // row - key = base - (mb*32 + jj*8 + i)
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int off = mb * 32 + jj * 8 + i;
        const bool vis = is_lm ? (key0 + g2 * 4 + off < lmc) : ((unsigned)(base - off) < (unsigned)w);
        s[mb][jj * 4 + i] = vis ? s[mb][jj * 4 + i] : -INFINITY;
      }
    }
  }
}

// Slots g2*8+0..3 <-> keys kk*16+g2*4+0..3, g2*8+4..7 <-> keys kk*16+8+g2*4+0..3.
// exp2(s*c2 + nm) of the tile's 32 scores of this lane, in pack order
// (p[kk*8 + j]: see the slot map above), and their float32 sum.
__device__ __forceinline__ float exp_tile(const f32x16* s, float c2, float nm, float* p) {
  float t[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int mb = kk >> 1;
    const int j0 = (kk & 1) * 2;
    float* q = p + kk * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      q[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mb][j0 * 4 + i], c2, nm));
      q[4 + i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mb][(j0 + 1) * 4 + i], c2, nm));
    }
    t[kk] = ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]));
  }
  return (t[0] + t[1]) + (t[2] + t[3]);
}

// Online softmax of one tile's scores: forms P = exp2(s*c2 - m) against the
// row's reference max m, packed to bf16 as the B operand of O^T += V^T P^T.
// m is raised only when it has fallen too far behind: when some lane's sum
// of the tile's P exceeds 2^8 (an overflow to +inf included, as on the first
// tile, where m starts at -1e30).  That tile is then redone against the row
// max, with O and the sums rescaled.  Either way every P of a tile, and so
// its sum, stays at most 2^8, and O and the sums share one reference --
// exact, whatever m is.  The common case costs one compare on top of the
// float32 sum that LSE needs anyway; the row max (over both lanes) is formed
// only when the tile is redone.
template <int D>
__device__ __forceinline__ void softmax_tile(const f32x16* s, float c2, RowState<D>& st, bf16x8* pf) {
  float p[32];
  float tsum = exp_tile(s, c2, -st.m, p);
  if (__any(!(tsum <= kMaxTileSum))) {
    // Two chains of three-input maxima (v_max3_f32): 17 instructions for 32 scores.
    float a = fmaxf(fmaxf(s[0][0], s[0][1]), s[0][2]);
    float b = fmaxf(fmaxf(s[1][0], s[1][1]), s[1][2]);
#pragma unroll
    for (int e = 3; e < 15; e += 2) {
      a = fmaxf(fmaxf(a, s[0][e]), s[0][e + 1]);
      b = fmaxf(fmaxf(b, s[1][e]), s[1][e + 1]);
    }
    const float lane_max = fmaxf(fmaxf(a, s[0][15]), fmaxf(b, s[1][15]));
    const float m_new = fmaxf(st.m, half_max(lane_max) * c2);
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
    st.m = m_new;
    st.l *= alpha;
    st.ls *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) st.o[db] *= alpha;
    tsum = exp_tile(s, c2, -st.m, p);
  }
  st.ls += tsum;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const float* q = p + kk * 8;
    const uint32_t w0 = cvt_pk(q[0], q[1]);
    const uint32_t w1 = cvt_pk(q[2], q[3]);
    const uint32_t w2 = cvt_pk(q[4], q[5]);
    const uint32_t w3 = cvt_pk(q[6], q[7]);
    st.l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w0), ones, st.l, false);
    st.l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w1), ones, st.l, false);
    st.l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w2), ones, st.l, false);
    st.l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w3), ones, st.l, false);
    pf[kk] = __builtin_bit_cast(bf16x8, u32x4{w0, w1, w2, w3});
  }
}

// The matrix-core work of one step: optionally O^T += V^T P^T for one tile
// (PV) and S^T = K Q^T for another (QK), as one unrolled stream of operand
// fragments read from LDS four fragments ahead of the MFMA consuming them,
// in exactly this order (a scheduling barrier after every step).
// Consecutive MFMAs use independent accumulators.
template <int D, bool PV, bool QK>
__device__ __forceinline__ void mma_phase(const unsigned char* vt, const unsigned char* kt, const Frag<D>& fr,
                                          const bf16x8* qf, const bf16x8* pf, f32x16* o, f32x16* s) {
  using SM = Smem<D>;
  constexpr int DB = D / 32;
  constexpr int KS = D / 16;
  constexpr int NPV = PV ? 4 * DB : 0;  // (kk, db), db fastest
  constexpr int NQK = QK ? 2 * KS : 0;  // (ks, mb), mb fastest
  constexpr int N = NPV + NQK;
  constexpr int W = 4;                  // fragments in flight
  u32x4 f[N];
  auto load = [&](int i) -> u32x4 {
    if (i < NPV) {
      const int kk = i / DB, db = i % DB;
      const unsigned char* p = vt + fr.v[db] + kk * 16 * SM::RB;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)p);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(p + 8 * SM::RB));
      const auto a = __builtin_bit_cast(u32x2, lo);
      const auto c = __builtin_bit_cast(u32x2, hi);
      return u32x4{a[0], a[1], c[0], c[1]};
    }
    const int q = i - NPV;
    const int ks = q / 2, mb = q % 2;
    return *reinterpret_cast<const u32x4*>(kt + fr.k[ks] + mb * 32 * SM::RB);
  };
  if constexpr (QK) {
    s[0] = f32x16{};
    s[1] = f32x16{};
  }
#pragma unroll
  for (int i = 0; i < W && i < N; ++i) f[i] = load(i);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (i + W < N) f[i + W] = load(i + W);
    const bf16x8 a = __builtin_bit_cast(bf16x8, f[i]);
    if (i < NPV) {
      const int kk = i / DB, db = i % DB;
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kk], o[db], 0, 0, 0);
    } else {
      const int q = i - NPV;
      const int ks = q / 2, mb = q % 2;
      s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[mb], 0, 0, 0);
    }
    // Keep this order: the compiler would otherwise pull the reads in to just
    // ahead of their MFMA (exposing the LDS latency at every step) and mix
    // the softmax's vector work into the PV stream.  Whole phases of one
    // kind per wavefront interleave better with the other wavefront on the
    // SIMD (about 2.5% faster on the 128K workload, bit-identical output).
    __builtin_amdgcn_sched_barrier(0);
  }
}

// O = O_acc / sum(bf16 P), LSE = (m + log2 sum(P)) ln 2.  Called by every
// thread of the workgroup after the walk's last barrier, when no wavefront
// reads the tile buffers any more (bf16 rows are staged there).  O, LSE and
// Q are touched once, so they carry the non-temporal hint and leave the L2
// to the K/V tiles that the walks of neighbouring query tiles and heads read
// again.
template <int D, bool OUT_BF16>
__device__ __forceinline__ void store_rows(const RowState<D>& st, int wr0, int lane, int wave, int n,
                                           size_t q_off, size_t lse_off, unsigned char* smem,
                                           void* __restrict__ Out, float* __restrict__ LSE) {
  const int r32 = lane & 31;
  const int g2 = lane >> 5;
  const int row = wr0 + r32;
  const float lt = half_sum(st.l);
  const float lst = half_sum(st.ls);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  if constexpr (OUT_BF16) {
    store_rows_bf16_nt<D>(st.o, inv, smem + wave * 32 * (D * 2 + 16), lane,
                          static_cast<uint16_t*>(Out) + q_off + (size_t)wr0 * D, n - wr0);
  } else if (row < n) {
    const size_t base = q_off + (size_t)row * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int dcol = db * 32 + jj * 8 + g2 * 4;
        *reinterpret_cast<f32x4*>(static_cast<float*>(Out) + base + dcol) =
            f32x4{st.o[db][jj * 4 + 0] * inv, st.o[db][jj * 4 + 1] * inv, st.o[db][jj * 4 + 2] * inv,
                  st.o[db][jj * 4 + 3] * inv};
      }
    }
  }
  if (LSE != nullptr && g2 == 0 && row < n) __builtin_nontemporal_store((st.m + log2f(lst)) * kLn2, LSE + lse_off + row);
}

// Everything a workgroup needs to walk the tiles of one query tile.
template <int D>
struct Walk {
  TileRange tr;
  int n_tiles;
  __amdgpu_buffer_rsrc_t rk, rv, rkl, rvl;  // window and landmark K/V of the KV head
  int n;

  __device__ void init(const uint16_t* K, const uint16_t* V, const uint16_t* Kb, const uint16_t* Vb, int b,
                       int Hkv, int kvh, int t, int n_, int w, int G, int L) {
    n = n_;
    tr = tile_range(t, BM, BN, n, w, G, L);
    n_tiles = tr.n_lm_tiles + (tr.kt_hi - tr.kt_lo + 1);
    const size_t kv_off = ((size_t)b * Hkv + kvh) * (size_t)n * D;
    rk = make_rsrc(K + kv_off, (uint32_t)n * D * 2u);
    rv = make_rsrc(V + kv_off, (uint32_t)n * D * 2u);
    rkl = rk;
    rvl = rv;
    if (G > 0) {
      const size_t lm_off = ((size_t)b * Hkv + kvh) * (size_t)G * D;
      rkl = make_rsrc(Kb + lm_off, (uint32_t)G * D * 2u);
      rvl = make_rsrc(Vb + lm_off, (uint32_t)G * D * 2u);
    }
  }
  __device__ bool is_lm(int it) const { return it < tr.n_lm_tiles; }
  // First key (landmark index or position) of tile it.  Past the last tile:
  // n, beyond the window buffer, so loads of it are range-checked away and
  // touch no memory.
  __device__ int key0(int it) const {
    return it >= n_tiles ? n : (it < tr.n_lm_tiles ? it * BN : (tr.kt_lo + it - tr.n_lm_tiles) * BN);
  }
  __device__ __amdgpu_buffer_rsrc_t ksrc(int it) const { return is_lm(it) ? rkl : rk; }
  __device__ __amdgpu_buffer_rsrc_t vsrc(int it) const { return is_lm(it) ? rvl : rv; }
};

// Q fragments of one row (B operand of S^T = K Q^T).
template <int D>
__device__ __forceinline__ void load_q(const uint16_t* __restrict__ Q, size_t q_off, int row, int n, int g2,
                                       bf16x8* qf) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < n) v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Q + q_off + (size_t)row * D + ks * 16 + g2 * 8));
    qf[ks] = __builtin_bit_cast(bf16x8, v);
  }
}

// Zero the tile buffers once: rows the range check skips keep finite values.
template <int D>
__device__ __forceinline__ void zero_smem(unsigned char* smem, int tid, int nthreads) {
  for (int i = tid; i < Smem<D>::BYTES / 16; i += nthreads) {
    reinterpret_cast<u32x4*>(smem)[i] = u32x4{0u, 0u, 0u, 0u};
  }
}

// Wait for this wavefront's direct-to-LDS loads, then the workgroup barrier.
__device__ __forceinline__ void lds_loads_done_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0); other counters unconstrained
  __syncthreads();
}

// Per-wavefront constants of the walk.
struct TileCtx {
  int wr0, wr1, wlm_lo, wlm_hi, w, row, lmc, g2;
  bool live;
  float c2;
};

// One tile of the walk: issue the next tile's loads into the other buffer,
// then scores, mask, softmax and PV from buffer BUF (= it & 1).
template <int D, int BUF>
__device__ __forceinline__ void tile_step(int it, unsigned char* smem, const Stager<D>& sg, const Walk<D>& wk,
                                          const Frag<D>& fr, const bf16x8* qf, RowState<D>& st, const TileCtx& tc) {
  using SM = Smem<D>;
  sg.issue_k(wk.ksrc(it + 1), smem + SM::kbuf(BUF ^ 1), wk.key0(it + 1));
  sg.issue_v(wk.vsrc(it + 1), smem + SM::vbuf(BUF ^ 1), wk.key0(it + 1));
  const TileVis v = tile_vis(wk.is_lm(it), wk.key0(it), tc.wr0, tc.wr1, tc.wlm_lo, tc.wlm_hi, tc.w);
  if (tc.live && v.any) {
    f32x16 s[2];
    bf16x8 pf[4];
    mma_phase<D, false, true>(nullptr, smem + SM::kbuf(BUF), fr, qf, pf, st.o, s);
    if (!v.interior) mask_tile(s, wk.is_lm(it), wk.key0(it), tc.row, tc.lmc, tc.w, tc.g2);
    softmax_tile<D>(s, tc.c2, st, pf);
    mma_phase<D, true, false>(smem + SM::vbuf(BUF), nullptr, fr, qf, pf, st.o, s);
  }
  lds_loads_done_barrier();
}

// ---------------------------------------------------------------------------
// The kernel: 4 wavefronts own one 128-row query tile of one head.
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ Kb, const uint16_t* __restrict__ Vb, void* __restrict__ Out,
    float* __restrict__ LSE, int Hq, int Hkv, int n, int w, int G, int L, float c2, int T) {
  using SM = Smem<D>;
  __shared__ __align__(16) unsigned char smem[SM::BYTES];

  const int j = xcd_remap(blockIdx.x, gridDim.x);
  const int grp = Hq / Hkv;
  const int h_in = j % grp;
  int rest = j / grp;
  const int t = T - 1 - rest % T;
  rest /= T;
  const int kvh = rest % Hkv;
  const int b = rest / Hkv;
  const int h = kvh * grp + h_in;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_index(tid);
  const int r32 = lane & 31;
  const int g2 = lane >> 5;

  zero_smem<D>(smem, tid, kThreads);

  Walk<D> wk;
  wk.init(K, V, Kb, Vb, b, Hkv, kvh, t, n, w, G, L);
  const int n_tiles = wk.n_tiles;

  const int wr0 = wk.tr.r0 + wave * 32;
  const int wr1 = min(wr0 + 31, n - 1);
  const int row = wr0 + r32;
  const int lmc = lm_count(row, w, G, L);
  const int wlm_lo = lm_count(wr0, w, G, L);
  const int wlm_hi = wr0 <= n - 1 ? lm_count(wr1, w, G, L) : 0;
  const bool live = wr0 <= n - 1;

  const size_t q_off = ((size_t)b * Hq + h) * (size_t)n * D;
  bf16x8 qf[D / 16];
  load_q<D>(Q, q_off, row, n, g2, qf);

  RowState<D> st;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) st.o[db] = f32x16{};
  st.m = -1e30f;
  st.l = 0.f;
  st.ls = 0.f;

  Stager<D> sg;
  sg.init(tid);
  Frag<D> fr;
  fr.init(lane);
  __syncthreads();  // zeroed buffers in place before any load lands

  sg.issue_k(wk.ksrc(0), smem + SM::kbuf(0), wk.key0(0));
  sg.issue_v(wk.vsrc(0), smem + SM::vbuf(0), wk.key0(0));
  lds_loads_done_barrier();

  // Two tiles per trip, so each one's LDS buffer is a compile-time offset
  // that the operand reads take as an immediate.
  const TileCtx tc{wr0, wr1, wlm_lo, wlm_hi, w, row, lmc, g2, live, c2};
  int it = 0;
  for (; it + 1 < n_tiles; it += 2) {
    tile_step<D, 0>(it, smem, sg, wk, fr, qf, st, tc);
    tile_step<D, 1>(it + 1, smem, sg, wk, fr, qf, st, tc);
  }
  if (it < n_tiles) tile_step<D, 0>(it, smem, sg, wk, fr, qf, st, tc);
  store_rows<D, OUT_BF16>(st, wr0, lane, wave, n, q_off, ((size_t)b * Hq + h) * n, smem, Out, LSE);
}

// ---------------------------------------------------------------------------
// Block-sparse lists: query tile t of head h visits the 64-key blocks listed
// for it (block index kb covers keys kb*64 .. kb*64+63, clipped at n),
// optionally causal, with the same tile pipeline as the window walk.  An
// index outside [0, ceil(n/64)) loads nothing and is skipped.
template <int D>
struct ListWalk {
  const int32_t* idx;
  int count, nkb, n;
  __amdgpu_buffer_rsrc_t rk, rv;
  // First key of list entry it; n (no tile) past the end or out of range.
  __device__ int key0(int it) const {
    if (it >= count) return n;
    const int kb = idx[it];
    return (kb >= 0 && kb < nkb) ? kb * BN : n;
  }
};

// -inf on every score of tile key0 that this lane's row does not see.
__device__ __forceinline__ void mask_list_tile(f32x16* s, int key0, int row, int n, bool causal, int g2) {
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = key0 + mb * 32 + jj * 8 + g2 * 4 + i;
        const bool vis = key < n && (!causal || key <= row);
        s[mb][jj * 4 + i] = vis ? s[mb][jj * 4 + i] : -INFINITY;
      }
    }
  }
}

template <int D, int BUF>
__device__ __forceinline__ void list_tile_step(int key_cur, int key_nxt, bool causal, unsigned char* smem,
                                               const Stager<D>& sg, const ListWalk<D>& wk, const Frag<D>& fr,
                                               const bf16x8* qf, RowState<D>& st, const TileCtx& tc) {
  using SM = Smem<D>;
  sg.issue_k(wk.rk, smem + SM::kbuf(BUF ^ 1), key_nxt);
  sg.issue_v(wk.rv, smem + SM::vbuf(BUF ^ 1), key_nxt);
  const bool any = key_cur < wk.n && (!causal || key_cur <= tc.wr1);
  const bool interior = key_cur + BN <= wk.n && (!causal || key_cur + BN - 1 <= tc.wr0);
  if (tc.live && any) {
    f32x16 s[2];
    bf16x8 pf[4];
    mma_phase<D, false, true>(nullptr, smem + SM::kbuf(BUF), fr, qf, pf, st.o, s);
    if (!interior) mask_list_tile(s, key_cur, tc.row, wk.n, causal, tc.g2);
    softmax_tile<D>(s, tc.c2, st, pf);
    mma_phase<D, true, false>(smem + SM::vbuf(BUF), nullptr, fr, qf, pf, st.o, s);
  }
  lds_loads_done_barrier();
}

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_list_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ indices, int max_blocks, int causal_i,
    void* __restrict__ Out, float* __restrict__ LSE, int Hq, int Hkv, int n, float c2, int T) {
  using SM = Smem<D>;
  __shared__ __align__(16) unsigned char smem[SM::BYTES];

  const int j = xcd_remap(blockIdx.x, gridDim.x);
  const int grp = Hq / Hkv;
  const int h_in = j % grp;
  int rest = j / grp;
  const int t = rest % T;
  rest /= T;
  const int kvh = rest % Hkv;
  const int b = rest / Hkv;
  const int h = kvh * grp + h_in;
  const bool causal = causal_i != 0;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_index(tid);
  const int r32 = lane & 31;
  const int g2 = lane >> 5;

  zero_smem<D>(smem, tid, kThreads);

  ListWalk<D> wk;
  const size_t list = ((size_t)b * Hq + h) * T + t;
  const int cnt = counts[list];
  wk.count = cnt < 0 ? 0 : (cnt > max_blocks ? max_blocks : cnt);
  wk.idx = indices + list * (size_t)max_blocks;
  wk.nkb = (n + BN - 1) / BN;
  wk.n = n;
  const size_t kv_off = ((size_t)b * Hkv + kvh) * (size_t)n * D;
  wk.rk = make_rsrc(K + kv_off, (uint32_t)n * D * 2u);
  wk.rv = make_rsrc(V + kv_off, (uint32_t)n * D * 2u);

  const int wr0 = t * BM + wave * 32;
  const int wr1 = min(wr0 + 31, n - 1);
  const int row = wr0 + r32;
  const bool live = wr0 <= n - 1;

  const size_t q_off = ((size_t)b * Hq + h) * (size_t)n * D;
  bf16x8 qf[D / 16];
  load_q<D>(Q, q_off, row, n, g2, qf);

  RowState<D> st;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) st.o[db] = f32x16{};
  st.m = -1e30f;
  st.l = 0.f;
  st.ls = 0.f;

  Stager<D> sg;
  sg.init(tid);
  Frag<D> fr;
  fr.init(lane);
  __syncthreads();  // zeroed buffers in place before any load lands

  int key_cur = wk.key0(0);
  int key_nxt = wk.key0(1);
  sg.issue_k(wk.rk, smem + SM::kbuf(0), key_cur);
  sg.issue_v(wk.rv, smem + SM::vbuf(0), key_cur);
  lds_loads_done_barrier();

  // the list entry two ahead is read while the current tile computes
  const TileCtx tc{wr0, wr1, 0, 0, 0, row, 0, g2, live, c2};
  int it = 0;
  for (; it + 1 < wk.count; it += 2) {
    int key_2 = wk.key0(it + 2);
    list_tile_step<D, 0>(key_cur, key_nxt, causal, smem, sg, wk, fr, qf, st, tc);
    key_cur = key_nxt;
    key_nxt = key_2;
    key_2 = wk.key0(it + 3);
    list_tile_step<D, 1>(key_cur, key_nxt, causal, smem, sg, wk, fr, qf, st, tc);
    key_cur = key_nxt;
    key_nxt = key_2;
  }
  if (it < wk.count) list_tile_step<D, 0>(key_cur, key_nxt, causal, smem, sg, wk, fr, qf, st, tc);
  store_rows<D, OUT_BF16>(st, wr0, lane, wave, n, q_off, ((size_t)b * Hq + h) * n, smem, Out, LSE);
}

template <int D, bool OUT_BF16>
hipError_t launch_list_t(const msa_attn_desc& d, const int32_t* counts, const int32_t* indices, int max_blocks,
                         int causal, const void* Q, const void* K, const void* V, void* O, float* LSE,
                         hipStream_t stream) {
  const int n = d.seq_len;
  const int T = (n + BM - 1) / BM;
  const long long wgs = (long long)d.batch * d.heads_q * T;
  hipLaunchKernelGGL((attn_fwd_list_kernel<D, OUT_BF16>), dim3((unsigned)wgs), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K),
                     static_cast<const uint16_t*>(V), counts, indices, max_blocks, causal, O, LSE, d.heads_q,
                     d.heads_kv, n, d.scale * kLog2e, T);
  return hipGetLastError();
}

template <int D, bool OUT_BF16>
hipError_t launch_t(const msa_attn_desc& d, const void* Q, const void* K, const void* V,
                    const void* Kb, const void* Vb, void* O, float* LSE, hipStream_t stream) {
  const int n = d.seq_len;
  const int T = (n + BM - 1) / BM;
  const int G = d.num_landmarks;
  const int L = G > 0 ? n / G : 1;
  const auto q = static_cast<const uint16_t*>(Q);
  const auto k = static_cast<const uint16_t*>(K);
  const auto v = static_cast<const uint16_t*>(V);
  const auto kb = static_cast<const uint16_t*>(Kb);
  const auto vb = static_cast<const uint16_t*>(Vb);
  const long long wgs = (long long)d.batch * d.heads_q * T;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, OUT_BF16>), dim3((unsigned)wgs), dim3(kThreads), 0, stream, q, k,
                     v, kb, vb, O, LSE, d.heads_q, d.heads_kv, n, d.window, G, L, d.scale * kLog2e, T);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_list_bf16(const msa_attn_desc& d, const int32_t* counts, const int32_t* indices,
                                 int max_blocks, int causal, const void* Q, const void* K, const void* V, void* O,
                                 float* LSE, hipStream_t stream) {
  const bool ob = d.out_dtype == MSA_DTYPE_BF16;
  if (d.head_dim == 128) {
    return ob ? launch_list_t<128, true>(d, counts, indices, max_blocks, causal, Q, K, V, O, LSE, stream)
              : launch_list_t<128, false>(d, counts, indices, max_blocks, causal, Q, K, V, O, LSE, stream);
  }
  return ob ? launch_list_t<64, true>(d, counts, indices, max_blocks, causal, Q, K, V, O, LSE, stream)
            : launch_list_t<64, false>(d, counts, indices, max_blocks, causal, Q, K, V, O, LSE, stream);
}

hipError_t launch_attn_bf16(const msa_attn_desc& d, const void* Q, const void* K, const void* V,
                            const void* Kbar, const void* Vbar, void* O, float* LSE,
                            hipStream_t stream) {
  const bool ob = d.out_dtype == MSA_DTYPE_BF16;
  if (d.head_dim == 128) {
    return ob ? launch_t<128, true>(d, Q, K, V, Kbar, Vbar, O, LSE, stream)
              : launch_t<128, false>(d, Q, K, V, Kbar, Vbar, O, LSE, stream);
  }
  return ob ? launch_t<64, true>(d, Q, K, V, Kbar, Vbar, O, LSE, stream)
            : launch_t<64, false>(d, Q, K, V, Kbar, Vbar, O, LSE, stream);
}

}  // namespace msa
