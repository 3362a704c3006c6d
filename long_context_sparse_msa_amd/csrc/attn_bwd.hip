// Backward of the window + landmark attention for bf16 inputs on gfx950.
//
// What it computes: for an upstream gradient dO, the gradients of O with
// respect to Q, K and V through the single softmax over window keys and
// visible landmarks (the pattern of "Scaling GPU Cluster for Million Token
// Context", section "Why Sparse Attention Changes the Game"; the pages
// train at these lengths -- "Training at 1M+ Token Context ...", Flash
// Attention and Block-Sparse Flash Attention paragraphs -- without writing
// the backward out).  With P the normalised probabilities recomputed from
// the forward's LSE:
//   dP = dO V_vis^T,  D = rowsum(dO * O),  dS = P * (dP - D),
//   dQ = scale dS K_vis,  dK_vis = scale dS^T Q,  dV_vis = P^T dO,
// summed over the query heads of a KV group; each landmark's gradient goes
// to the L rows of its block with weight 1/L (a landmark is their mean).
//
// Kernels, in launch order:
//  1. bwd_dq_kernel: one 128-row query tile of one head per workgroup,
//     walking the same landmark and window key tiles as the forward.  It
//     first forms D = rowsum(dO * O) and the base-2 LSE of its rows and
//     stores them in a padded workspace array for the dK/dV kernels (rows
//     past n get LSE = +inf, so P = 0).  Per 64-key tile and wavefront (32
//     rows): S^T = K Q^T and dP^T = V dO^T on v_mfma_f32_32x32x16_bf16, P
//     and dS in registers (each lane holds 16 keys of one row), dQ^T +=
//     K^T dS^T with K^T read by ds_read_b64_tr_b16.
//  2. bwd_dkdv_kernel<landmarks>: one workgroup per 128 landmarks and one
//     segment of query rows; per-segment partial gradients of the landmarks
//     go to the workspace.
//  3. bwd_lm_reduce_kernel: sums the segments (fixed order, deterministic).
//  4. bwd_dkdv_kernel<window>: one workgroup per 128 keys of one KV head,
//     wavefront w owning keys 32w..32w+31, looping over every (query head of
//     the group, 32-row query block) that sees them.  S = Q K^T and
//     dP = dO V^T put one key per lane column, so P and dS are directly the
//     B operands of dV^T += dO^T P and dK^T += Q^T dS (dO^T and Q^T by
//     transpose reads).  The epilogue adds each row's share of its block's
//     landmark gradient.
// No atomics: every output element is written once by one workgroup.
//
// LDS tiles are row-major with 16-byte chunks permuted within a row.  Tiles
// read only row-per-lane use chunk c of row r at slot c ^ (r mod CH).  Tiles
// read both row-per-lane and by transpose reads use slot c ^ h(r), h(r) =
// 2*(r mod CH/2) + (r div CH/2 mod 2): a bijection over CH aligned rows, so
// 16 rows reading one chunk hit distinct slots, and with h(r)>>1 distinct
// over 4 aligned rows, so the 4 rows x 2 chunks a transpose read touches hit
// distinct slots.
#include "msa_device.hpp"
#include "msa_internal.hpp"
#include "msa_plan.hpp"

namespace msa {
namespace {

constexpr int kThreads = 256;
constexpr int BM = kBM_BF16;  // 128 query rows per dQ workgroup
constexpr int BN = kBN_BF16;  // 64 keys per dQ tile
constexpr int KB = 128;       // keys per dK/dV workgroup (4 wavefronts x 32)
constexpr int QB = 32;        // query rows per dK/dV step
constexpr int kPad = 128;     // the (LSE, D) array pads each head's rows to a multiple of this

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;

template <int D>
struct Sw {
  static constexpr int RB = 2 * D;
  static constexpr int CH = RB / 16;
  __device__ static constexpr int row(int r) { return r % CH; }
  __device__ static constexpr int both(int r) { return ((r % (CH / 2)) << 1) | ((r / (CH / 2)) & 1); }
  // Byte offset of (row r, dim d) in a tile with the row or the both swizzle.
  __device__ static constexpr uint32_t at_row(int r, int d) {
    return (uint32_t)(r * RB + (((d / 8) ^ row(r)) * 16) + (d % 8) * 2);
  }
  __device__ static constexpr uint32_t at_both(int r, int d) {
    return (uint32_t)(r * RB + (((d / 8) ^ both(r)) * 16) + (d % 8) * 2);
  }
};

// Direct-to-LDS loads of a ROWS x D bf16 tile by the 256 threads of a
// workgroup: instruction i of wavefront wv fills LDS bytes
// [i*4096 + wv*1024, +1024), lane l the 16 bytes at l*16.  Rows past the
// buffer end are skipped by the range check (their LDS keeps what it held).
template <int D, int ROWS>
struct TileLoader {
  using S = Sw<D>;
  static constexpr int BYTES = ROWS * S::RB;
  static constexpr int NI = BYTES / 4096;
  static_assert(NI >= 1 && BYTES % 4096 == 0, "tile is a multiple of 4 KB");
  uint32_t off[NI];
  int wv;
  __device__ void init(int tid, bool both) {
    wv = wave_index(tid);
    const int lane = tid & 63;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int q = (i * 4 + wv) * 64 + lane;
      const int r = q / S::CH, slot = q % S::CH;
      off[i] = (uint32_t)(r * S::RB + ((slot ^ (both ? S::both(r) : S::row(r))) * 16));
    }
  }
  __device__ void issue(__amdgpu_buffer_rsrc_t rsrc, unsigned char* tile, int row0) const {
    const uint32_t soff = (uint32_t)row0 * S::RB;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_ptr)(tile + i * 4096 + wv * 1024), 16, off[i], soff,
                                               0, 0);
    }
  }
};

__device__ __forceinline__ void wait_loads_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0); other counters unconstrained
  __syncthreads();
}

__device__ __forceinline__ void zero_lds(unsigned char* p, int bytes, int tid) {
  for (int i = tid; i < bytes / 16; i += kThreads) reinterpret_cast<u32x4*>(p)[i] = u32x4{0u, 0u, 0u, 0u};
}

// A 32-lane transpose-read operand: rows base .. base+3 (lo) and base+8 ..
// base+11 (hi) of a both-swizzled tile, at the dims this lane's group reads.
__device__ __forceinline__ bf16x8 tr_pair(const unsigned char* tile, uint32_t lo, uint32_t hi) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(tile + lo));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(tile + hi));
  const u32x2 x = __builtin_bit_cast(u32x2, a), y = __builtin_bit_cast(u32x2, b);
  return __builtin_bit_cast(bf16x8, u32x4{x[0], x[1], y[0], y[1]});
}

// Offsets of the transpose reads for dim block db (32 dims) and a 16-row
// step: within each 16-lane group, lane j points at row (g2*4 + j/4), dims
// db*32 + (g&1)*16 + 4*(j%4); the pair hands lane l the 8 rows
// {g2*4 + 0..3, 8 + g2*4 + 0..3} of dim db*32 + l%32, which is the operand
// slot order of a C-layout accumulator packed as B (slots g2*8+0..3 <-> rows
// g2*4+0..3, g2*8+4..7 <-> rows 8+g2*4+0..3).  Step kk adds 16 rows, which
// keeps the swizzle (its period divides 16).
template <int D>
struct TrOffsets {
  uint32_t lo[D / 32], hi[D / 32];
  __device__ void init(int lane) {
    const int g = lane >> 4, j = lane & 15;
    const int r = (g >> 1) * 4 + (j >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int d = db * 32 + (g & 1) * 16 + 4 * (j & 3);
      lo[db] = Sw<D>::at_both(r, d);
      hi[db] = Sw<D>::at_both(r + 8, d);
    }
  }
};

// Packs a C-layout score block (16 floats per lane: rows jj*8 + g2*4 + i)
// into the two B operands of the 16-row k-steps kk = 0, 1.
__device__ __forceinline__ void pack_b(const float* x, bf16x8* out) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int j0 = kk * 2;
    const uint32_t w0 = cvt_pk(x[j0 * 4 + 0], x[j0 * 4 + 1]);
    const uint32_t w1 = cvt_pk(x[j0 * 4 + 2], x[j0 * 4 + 3]);
    const uint32_t w2 = cvt_pk(x[(j0 + 1) * 4 + 0], x[(j0 + 1) * 4 + 1]);
    const uint32_t w3 = cvt_pk(x[(j0 + 1) * 4 + 2], x[(j0 + 1) * 4 + 3]);
    out[kk] = __builtin_bit_cast(bf16x8, u32x4{w0, w1, w2, w3});
  }
}

// ---------------------------------------------------------------------------
// 1. dQ: the forward's walk, with dP^T = V dO^T and dQ^T += K^T dS^T.
template <int D>
struct DqSmem {
  static constexpr int TILE = BN * Sw<D>::RB;
  static constexpr int BYTES = 4 * TILE;
  __device__ static constexpr int kbuf(int i) { return i * TILE; }
  __device__ static constexpr int vbuf(int i) { return (2 + i) * TILE; }
};

// The tiles one query tile visits (landmark tiles, then window tiles) and
// their sources.  Past the last tile key0 is n, beyond the window buffer,
// so its loads are range-checked away.  (A struct method rather than a
// lambda in the kernel: with the load builtins inside a lambda the host
// pass drops the kernel's launch stub.)
template <int D>
struct DqWalk {
  TileRange tr;
  int n_tiles, n;
  __amdgpu_buffer_rsrc_t rk, rv, rkl, rvl;
  TileLoader<D, BN> ldk, ldv;
  __device__ bool is_lm(int it) const { return it < tr.n_lm_tiles; }
  __device__ int key0(int it) const {
    return it >= n_tiles ? n : (it < tr.n_lm_tiles ? it * BN : (tr.kt_lo + it - tr.n_lm_tiles) * BN);
  }
  __device__ void issue(unsigned char* smem, int it, int buf) const {
    const bool lm = is_lm(it);
    ldk.issue(lm ? rkl : rk, smem + DqSmem<D>::kbuf(buf), key0(it));
    ldv.issue(lm ? rvl : rv, smem + DqSmem<D>::vbuf(buf), key0(it));
  }
};

// Per-wavefront constants of the dQ walk.
struct DqCtx {
  int wr0, wr1, wlm_lo, wlm_hi, w, row, lmc, g2;
  bool live;
  float c2, nl2, Drow;
};

// One tile of the dQ walk: issue the next tile's loads into the other
// buffer, then S^T, dP^T, dS^T and dQ^T += K^T dS^T from buffer BUF.  BUF is
// a compile-time constant, so every operand read takes its tile offset as an
// immediate (a runtime buffer index costs one address add per read).
template <int D, int BUF>
__device__ __forceinline__ void dq_step(int it, unsigned char* smem, const DqWalk<D>& wk, const DqCtx& c,
                                        const bf16x8* qf, const bf16x8* df, const uint32_t* koff,
                                        const uint32_t* voff, const TrOffsets<D>& tro, f32x16* dq) {
  using SM = DqSmem<D>;
  using S = Sw<D>;
  constexpr int KS = D / 16, DB = D / 32;
  const int wr0 = c.wr0, wr1 = c.wr1, wlm_lo = c.wlm_lo, wlm_hi = c.wlm_hi, w = c.w, row = c.row, lmc = c.lmc;
  const int g2 = c.g2;
  const bool live = c.live;
  const float c2 = c.c2, nl2 = c.nl2, Drow = c.Drow;
  wk.issue(smem, it + 1, BUF ^ 1);
  const bool is_lm = wk.is_lm(it);
  const int key0 = wk.key0(it);
  bool any, interior;
  if (is_lm) {
    any = key0 < wlm_hi;
    interior = key0 + BN <= wlm_lo;
  } else {
    any = key0 <= wr1 && key0 + BN - 1 >= wr0 - w + 1;
    interior = key0 + BN - 1 <= wr0 && key0 >= wr1 - w + 1;
  }
  if (live && any) {
    const unsigned char* kt = smem + SM::kbuf(BUF);
    const unsigned char* vt = smem + SM::vbuf(BUF);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kt + koff[ks] + mb * 32 * S::RB);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s, 0, 0, 0);
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(vt + voff[ks] + mb * 32 * S::RB);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, df[ks], dp, 0, 0, 0);
      }
      // Edge tiles only (a wavefront-uniform branch): scores this lane's row
      // does not see become -inf, so P = exp2(-inf) = 0 below.  (A select
      // around the exponential instead compiles to one divergent branch per
      // element; the empty volatile asm keeps the compiler from turning this
      // branch into selects executed on every tile.)
      if (!interior) {
        asm volatile("");
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = key0 + mb * 32 + (e / 4) * 8 + g2 * 4 + e % 4;
          const bool vis = is_lm ? key < lmc : (unsigned)(row - key) < (unsigned)w;
          s[e] = vis ? s[e] : -INFINITY;
        }
      }
      float ds[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) ds[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], c2, nl2)) * (dp[e] - Drow);
      bf16x8 dsf[2];
      pack_b(ds, dsf);
#pragma unroll
      for (int kl = 0; kl < 2; ++kl) {
        const int rows0 = (mb * 2 + kl) * 16;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x8 a = tr_pair(kt + rows0 * S::RB, tro.lo[db], tro.hi[db]);
          dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsf[kl], dq[db], 0, 0, 0);
        }
      }
    }
  }
  wait_loads_barrier();
}

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ Kb, const uint16_t* __restrict__ Vb, const uint16_t* __restrict__ dO,
    const uint16_t* __restrict__ O, const float* __restrict__ LSE, float2* __restrict__ LD, void* __restrict__ dQ, int Hq, int Hkv, int n, int n_pad, int w, int G, int L,
    float c2, float scale, int T) {
  using SM = DqSmem<D>;
  using S = Sw<D>;
  constexpr int KS = D / 16, DB = D / 32;
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

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index(tid);
  const int r32 = lane & 31, g2 = lane >> 5;
  zero_lds(smem, SM::BYTES, tid);

  DqWalk<D> wk;
  wk.tr = tile_range(t, BM, BN, n, w, G, L);
  wk.n_tiles = wk.tr.n_lm_tiles + (wk.tr.kt_hi - wk.tr.kt_lo + 1);
  wk.n = n;
  const size_t kv_off = ((size_t)b * Hkv + kvh) * (size_t)n * D;
  wk.rk = make_rsrc(K + kv_off, (uint32_t)n * D * 2u);
  wk.rv = make_rsrc(V + kv_off, (uint32_t)n * D * 2u);
  wk.rkl = wk.rk;
  wk.rvl = wk.rv;
  if (G > 0) {
    const size_t lm_off = ((size_t)b * Hkv + kvh) * (size_t)G * D;
    wk.rkl = make_rsrc(Kb + lm_off, (uint32_t)G * D * 2u);
    wk.rvl = make_rsrc(Vb + lm_off, (uint32_t)G * D * 2u);
  }
  wk.ldk.init(tid, true);
  wk.ldv.init(tid, false);

  const int wr0 = wk.tr.r0 + wave * 32;
  const int wr1 = min(wr0 + 31, n - 1);
  const int row = wr0 + r32;
  const bool live = wr0 <= n - 1;
  const int lmc = lm_count(row, w, G, L);
  const int wlm_lo = lm_count(wr0, w, G, L);
  const int wlm_hi = live ? lm_count(wr1, w, G, L) : 0;

  const size_t q_off = ((size_t)b * Hq + h) * (size_t)n * D;
  bf16x8 qf[KS], df[KS];  // B operands: column = this lane's row, k = dims ks*16 + g2*8 .. +7
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 a = {0u, 0u, 0u, 0u}, c = {0u, 0u, 0u, 0u};
    if (row < n) {
      a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Q + q_off + (size_t)row * D + ks * 16 + g2 * 8));
      c = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(dO + q_off + (size_t)row * D + ks * 16 + g2 * 8));
    }
    qf[ks] = __builtin_bit_cast(bf16x8, a);
    df[ks] = __builtin_bit_cast(bf16x8, c);
  }
  // D = rowsum(dO * O) over this lane's half of the dims and its partner's
  // (lane l^32), and the base-2 LSE; both kept for the dK/dV kernels in the
  // padded array (every row < n_pad belongs to exactly one lane with g2 = 0)
  float dsum = 0.f;
  if (row < n) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 o = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(O + q_off + (size_t)row * D + ks * 16 + g2 * 8));
      const u32x4 g = __builtin_bit_cast(u32x4, df[ks]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dsum = fmaf(bf16_bits_to_f32(o[e] & 0xffffu), bf16_bits_to_f32(g[e] & 0xffffu), dsum);
        dsum = fmaf(bf16_bits_to_f32(o[e] >> 16), bf16_bits_to_f32(g[e] >> 16), dsum);
      }
    }
  }
  const float Drow = half_sum(dsum);
  const float lse2 = row < n ? LSE[((size_t)b * Hq + h) * n + row] * kLog2e : INFINITY;
  if (g2 == 0) LD[((size_t)b * Hq + h) * n_pad + row] = float2{lse2, Drow};  // row < n_pad always
  const float nl2 = -lse2;

  // operand offsets: K rows (both swizzle) and V rows (row swizzle) for
  // S^T = K Q^T and dP^T = V dO^T: row r32 (+32 per key half), chunk ks*2+g2
  uint32_t koff[KS], voff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    koff[ks] = S::at_both(r32, ks * 16 + g2 * 8);
    voff[ks] = S::at_row(r32, ks * 16 + g2 * 8);
  }
  TrOffsets<D> tro;
  tro.init(lane);

  f32x16 dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dq[db] = f32x16{};

  __syncthreads();  // zeroed tiles in place before any load lands
  wk.issue(smem, 0, 0);
  wait_loads_barrier();

  const DqCtx ctx{wr0, wr1, wlm_lo, wlm_hi, w, row, lmc, g2, live, c2, nl2, Drow};
  int it = 0;
  for (; it + 1 < wk.n_tiles; it += 2) {
    dq_step<D, 0>(it, smem, wk, ctx, qf, df, koff, voff, tro, dq);
    dq_step<D, 1>(it + 1, smem, wk, ctx, qf, df, koff, voff, tro, dq);
  }
  if (it < wk.n_tiles) dq_step<D, 0>(it, smem, wk, ctx, qf, df, koff, voff, tro, dq);

  // dQ is written once: bf16 rows leave through the (now idle) tile buffers
  // as whole lines, past the L2 that keeps the K/V tiles.
  if constexpr (OUT_BF16) {
    store_rows_bf16_nt<D>(dq, scale, smem + wave * 32 * (D * 2 + 16), lane,
                          static_cast<uint16_t*>(dQ) + q_off + (size_t)wr0 * D, n - wr0);
  } else if (row < n) {
    const size_t base = q_off + (size_t)row * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int dcol = db * 32 + jj * 8 + g2 * 4;
        *reinterpret_cast<f32x4*>(static_cast<float*>(dQ) + base + dcol) =
            f32x4{dq[db][jj * 4 + 0], dq[db][jj * 4 + 1], dq[db][jj * 4 + 2], dq[db][jj * 4 + 3]} * scale;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 3-5. dK, dV: key-tile parallel.
template <int D>
struct KvSmem {
  using S = Sw<D>;
  static constexpr int VT = KB * S::RB;   // the workgroup's V rows
  static constexpr int QT = QB * S::RB;   // one query block of Q or dO
  static constexpr int LDB = QB * 8;      // (lse2, D) of the block's rows
  static constexpr int STAGE = 2 * QT + LDB;
  static constexpr int BYTES = VT + 2 * STAGE;
  __device__ static constexpr int stage(int i) { return VT + i * STAGE; }
  __device__ static constexpr int qbuf(int i) { return stage(i); }
  __device__ static constexpr int obuf(int i) { return stage(i) + QT; }
  __device__ static constexpr int ldbuf(int i) { return stage(i) + 2 * QT; }
};

struct KvArgs {
  const uint16_t *Q, *K, *V, *Kb, *Vb, *dO;
  const float2* LD;
  float* part;       // landmark partials [seg][B*Hkv][G][2][D]
  const float* lmg;  // reduced landmark gradients [B*Hkv][G][2][D] (dK already scaled)
  void *dK, *dV;
  int B, Hq, Hkv, n, n_pad, w, G, L, nkt, nlt, nseg, seg;
  float c2, scale;
};

// Loads of a dK/dV workgroup: its V rows once (row swizzle), then per (query
// head, 32-row block) step the Q and dO rows (both swizzle) and the rows'
// (lse2, D) pairs.  (The loads are issued from methods of this struct: with
// a loader's method called straight from the kernel body, the host pass of
// this toolchain dropped the launch stubs of all but one instantiation.)
template <int D>
struct KvStager {
  TileLoader<D, QB> ldq;
  TileLoader<D, KB> ldv;
  __device__ void issue_v(__amdgpu_buffer_rsrc_t rv, unsigned char* smem, int key0) const {
    ldv.issue(rv, smem, key0);
  }
  int b, kvh, grp, qb_lo, nqb, n_it, wave, lane;
  __device__ void issue(const KvArgs& A, unsigned char* smem, int it, int buf) const {
    if (it >= n_it) return;
    const int h = kvh * grp + it / nqb;
    const int q0 = (qb_lo + it % nqb) * QB;
    const size_t qo = ((size_t)b * A.Hq + h) * (size_t)A.n * D;
    ldq.issue(make_rsrc(A.Q + qo, (uint32_t)A.n * D * 2u), smem + KvSmem<D>::qbuf(buf), q0);
    ldq.issue(make_rsrc(A.dO + qo, (uint32_t)A.n * D * 2u), smem + KvSmem<D>::obuf(buf), q0);
    if (wave == 0 && lane < QB / 2) {
      const float2* src = A.LD + ((size_t)b * A.Hq + h) * A.n_pad + q0;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(src, QB * 8), (lds_void_ptr)(smem + KvSmem<D>::ldbuf(buf)),
                                               16, (uint32_t)lane * 16, 0, 0, 0);
    }
  }
};

// One query block of the dK/dV walk: issue the next block's loads into the
// other buffer, then S, dP, dS and dV^T += dO^T P, dK^T += Q^T dS from buffer
// BUF (a compile-time constant, so every operand read takes its offset as an
// immediate).
template <int D, bool LM, int BUF>
__device__ __forceinline__ void kv_step(int it, const KvArgs& A, const KvStager<D>& st, unsigned char* smem,
                                        int k0, int key, int thr_lane, int g2, const bf16x8* kf,
                                        const uint32_t* qoff, const uint32_t* voff, const TrOffsets<D>& tro,
                                        f32x16* dk, f32x16* dv) {
  using SM = KvSmem<D>;
  using S = Sw<D>;
  constexpr int KS = D / 16, DB = D / 32;
  st.issue(A, smem, it + 1, BUF ^ 1);
  const int q0 = (st.qb_lo + it % st.nqb) * QB;
  bool any, interior;
  if constexpr (LM) {
    const int thr_lo = (k0 + 1) * A.L - 1 + A.w;
    const int thr_hi = (k0 + 32) * A.L - 1 + A.w;
    any = k0 < A.G && q0 + QB - 1 >= thr_lo;
    interior = k0 + 31 < A.G && q0 >= thr_hi;
  } else {
    any = q0 + QB - 1 >= k0 && q0 <= k0 + 31 + A.w - 1;
    interior = q0 >= k0 + 31 && q0 + QB - 1 <= k0 + A.w - 1;
  }
  if (any) {
    const unsigned char* qt = smem + SM::qbuf(BUF);
    const unsigned char* ot = smem + SM::obuf(BUF);
    const float* ldt = reinterpret_cast<const float*>(smem + SM::ldbuf(BUF));
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 qa = *reinterpret_cast<const bf16x8*>(qt + qoff[ks]);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[ks], s, 0, 0, 0);
      const bf16x8 oa = *reinterpret_cast<const bf16x8*>(ot + qoff[ks]);
      const bf16x8 vb = *reinterpret_cast<const bf16x8*>(smem + voff[ks]);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, vb, dp, 0, 0, 0);
    }
    // edge blocks only (wavefront-uniform; the empty volatile asm keeps it a
    // branch): unseen scores become -inf, so P = exp2(-inf) = 0 below
    // (padding rows past n have lse2 = +inf)
    if (!interior) {
      // rel = the lane's first row minus its key (minus the landmark's first
      // seeing row), made opaque so that the per-element row offsets stay
      // immediates instead of 16 loop-invariant registers
      int rel = q0 + g2 * 4 - (LM ? thr_lane : key);
      asm volatile("" : "+v"(rel));
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int d = rel + (e / 4) * 8 + e % 4;  // qrow - key (qrow - thr_lane)
        const bool vis = LM ? d >= 0 : (unsigned)d < (unsigned)A.w;
        s[e] = vis ? s[e] : -INFINITY;
      }
    }
    // rows jj*8 + g2*4 + i of the block: (lse2, D) pairs, 32 bytes per jj
    float p[16], ds[16];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int rb = jj * 8 + g2 * 4;
      const f32x4 a = *reinterpret_cast<const f32x4*>(ldt + rb * 2);
      const f32x4 c = *reinterpret_cast<const f32x4*>(ldt + rb * 2 + 4);
      const float l2[4] = {a[0], a[2], c[0], c[2]};
      const float dd[4] = {a[1], a[3], c[1], c[3]};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = jj * 4 + i;
        p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], A.c2, -l2[i]));
        ds[e] = p[e] * (dp[e] - dd[i]);
      }
    }
    bf16x8 pf[2], dsf[2];
    pack_b(p, pf);
    pack_b(ds, dsf);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8 oa = tr_pair(ot + kk * 16 * S::RB, tro.lo[db], tro.hi[db]);
        dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, pf[kk], dv[db], 0, 0, 0);
        const bf16x8 qa = tr_pair(qt + kk * 16 * S::RB, tro.lo[db], tro.hi[db]);
        dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, dsf[kk], dk[db], 0, 0, 0);
      }
    }
  }
  wait_loads_barrier();
}

template <int D, bool LM, bool OUT_BF16>
__global__ __launch_bounds__(kThreads, 2) void bwd_dkdv_kernel(KvArgs A) {
  using SM = KvSmem<D>;
  using S = Sw<D>;
  constexpr int KS = D / 16, DB = D / 32;
  __shared__ __align__(16) unsigned char smem[SM::BYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index(tid);
  const int r32 = lane & 31, g2 = lane >> 5;
  const int grp = A.Hq / A.Hkv;

  // workgroup -> (b, kvh, tile[, segment]); consecutive tiles of one KV head
  // on one XCD share their query blocks in L2
  const int j = xcd_remap(blockIdx.x, gridDim.x);
  int tile, sg = 0, bk;
  if constexpr (LM) {
    sg = j % A.nseg;
    tile = (j / A.nseg) % A.nlt;
    bk = j / (A.nseg * A.nlt);
  } else {
    tile = j % A.nkt;
    bk = j / A.nkt;
  }
  const int b = bk / A.Hkv, kvh = bk % A.Hkv;
  const int key0 = tile * KB;          // first key / landmark of the workgroup
  const int k0 = key0 + wave * 32;     // first of this wavefront's
  const int key = k0 + r32;            // this lane's

  // query rows the workgroup visits: [r_lo, r_hi)
  int r_lo, r_hi;
  if constexpr (LM) {
    const int thr0 = (key0 + 1) * A.L - 1 + A.w;  // first row that sees landmark key0
    r_lo = max(sg * A.seg, thr0);
    r_hi = min(A.n, (sg + 1) * A.seg);
  } else {
    r_lo = key0;
    r_hi = min(A.n, key0 + KB - 1 + A.w);
  }
  const int qb_lo = r_lo / QB;
  const int nqb = r_hi > r_lo ? (r_hi - 1) / QB - qb_lo + 1 : 0;
  const int n_it = nqb * grp;

  // this lane's key (or landmark) row: K^T operand in registers, and the
  // first row that sees it (landmarks)
  const int nkeys = LM ? A.G : A.n;
  const uint16_t* kbase = LM ? A.Kb + (size_t)bk * A.G * D : A.K + (size_t)bk * A.n * D;
  const uint16_t* vbase = LM ? A.Vb + (size_t)bk * A.G * D : A.V + (size_t)bk * A.n * D;
  bf16x8 kf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (key < nkeys) v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + (size_t)key * D + ks * 16 + g2 * 8));
    kf[ks] = __builtin_bit_cast(bf16x8, v);
  }
  const int thr_lane = LM ? (key < A.G ? (key + 1) * A.L - 1 + A.w : 0x7fffffff) : 0;

  zero_lds(smem, SM::BYTES, tid);
  KvStager<D> st;
  st.ldv.init(tid, false);
  st.ldq.init(tid, true);
  st.b = b;
  st.kvh = kvh;
  st.grp = grp;
  st.qb_lo = qb_lo;
  st.nqb = nqb;
  st.n_it = n_it;
  st.wave = wave;
  st.lane = lane;
  uint32_t voff[KS], qoff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    voff[ks] = S::at_row(wave * 32 + r32, ks * 16 + g2 * 8);
    qoff[ks] = S::at_both(r32, ks * 16 + g2 * 8);
  }
  TrOffsets<D> tro;
  tro.init(lane);
  __syncthreads();

  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase, (uint32_t)nkeys * D * 2u);
  st.issue_v(rv, smem, key0);
  st.issue(A, smem, 0, 0);
  wait_loads_barrier();

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  int it = 0;
  for (; it + 1 < n_it; it += 2) {
    kv_step<D, LM, 0>(it, A, st, smem, k0, key, thr_lane, g2, kf, qoff, voff, tro, dk, dv);
    kv_step<D, LM, 1>(it + 1, A, st, smem, k0, key, thr_lane, g2, kf, qoff, voff, tro, dk, dv);
  }
  if (it < n_it) kv_step<D, LM, 0>(it, A, st, smem, k0, key, thr_lane, g2, kf, qoff, voff, tro, dk, dv);

  // lane (r32, g2) holds dims db*32 + jj*8 + g2*4 + i of key `key`
  if constexpr (LM) {
    if (key >= A.G) return;
    float* dst = A.part + (((size_t)sg * A.B * A.Hkv + bk) * A.G + key) * 2 * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int dcol = db * 32 + jj * 8 + g2 * 4;
        *reinterpret_cast<f32x4*>(dst + dcol) =
            f32x4{dk[db][jj * 4 + 0], dk[db][jj * 4 + 1], dk[db][jj * 4 + 2], dk[db][jj * 4 + 3]} * A.scale;
        *reinterpret_cast<f32x4*>(dst + D + dcol) =
            f32x4{dv[db][jj * 4 + 0], dv[db][jj * 4 + 1], dv[db][jj * 4 + 2], dv[db][jj * 4 + 3]};
      }
    }
  } else {
    if (key >= A.n) return;
    const float* lg = nullptr;
    float invL = 0.f;
    if (A.G > 0) {
      lg = A.lmg + ((size_t)bk * A.G + key / A.L) * 2 * D;
      invL = 1.0f / (float)A.L;
    }
    const size_t base = ((size_t)bk * A.n + key) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int dcol = db * 32 + jj * 8 + g2 * 4;
        f32x4 gk = f32x4{dk[db][jj * 4 + 0], dk[db][jj * 4 + 1], dk[db][jj * 4 + 2], dk[db][jj * 4 + 3]} * A.scale;
        f32x4 gv = f32x4{dv[db][jj * 4 + 0], dv[db][jj * 4 + 1], dv[db][jj * 4 + 2], dv[db][jj * 4 + 3]};
        if (lg != nullptr) {
          gk += *reinterpret_cast<const f32x4*>(lg + dcol) * invL;
          gv += *reinterpret_cast<const f32x4*>(lg + D + dcol) * invL;
        }
        if constexpr (OUT_BF16) {
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(A.dK) + base + dcol) =
              u32x2{cvt_pk(gk[0], gk[1]), cvt_pk(gk[2], gk[3])};
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(A.dV) + base + dcol) =
              u32x2{cvt_pk(gv[0], gv[1]), cvt_pk(gv[2], gv[3])};
        } else {
          *reinterpret_cast<f32x4*>(static_cast<float*>(A.dK) + base + dcol) = gk;
          *reinterpret_cast<f32x4*>(static_cast<float*>(A.dV) + base + dcol) = gv;
        }
      }
    }
  }
}

// 4. Landmark gradients: sum of the segments' partials, in segment order.
__global__ __launch_bounds__(256) void bwd_lm_reduce_kernel(const float* __restrict__ part, float* __restrict__ lmg,
                                                            long long per_seg, int nseg) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= per_seg) return;
  float acc = 0.f;
  for (int s = 0; s < nseg; ++s) acc += part[(size_t)s * per_seg + i];
  lmg[i] = acc;
}

template <int D, bool OUT_BF16>
hipError_t launch_bwd_t(const msa_attn_desc& d, const BwdLayout& lay, const void* Q, const void* K, const void* V,
                        const void* Kb, const void* Vb, const void* O, const float* LSE, const void* dO, void* ws,
                        void* dQ, void* dK, void* dV, hipStream_t stream) {
  const int n = d.seq_len, G = d.num_landmarks, L = G > 0 ? n / G : 1;
  const auto u16 = [](const void* p) { return static_cast<const uint16_t*>(p); };
  unsigned char* wsb = static_cast<unsigned char*>(ws);
  float2* LD = reinterpret_cast<float2*>(wsb + lay.ld_off);
  float* part = reinterpret_cast<float*>(wsb + lay.part_off);
  float* lmg = reinterpret_cast<float*>(wsb + lay.lmg_off);
  const float c2 = d.scale * kLog2e;

  hipError_t e;
  const int T = (n + BM - 1) / BM;
  hipLaunchKernelGGL((bwd_dq_kernel<D, OUT_BF16>), dim3((unsigned)((long long)d.batch * d.heads_q * T)),
                     dim3(kThreads), 0, stream, u16(Q), u16(K), u16(V), u16(Kb), u16(Vb), u16(dO), u16(O), LSE, LD, dQ,
                     d.heads_q, d.heads_kv, n, lay.n_pad, d.window, G, L, c2, d.scale, T);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  KvArgs A{u16(Q), u16(K), u16(V), u16(Kb), u16(Vb), u16(dO), LD, part, lmg, dK, dV,
           d.batch, d.heads_q, d.heads_kv, n, lay.n_pad, d.window, G, L,
           (n + KB - 1) / KB, (G + KB - 1) / KB, lay.nseg, lay.seg, c2, d.scale};
  const long long pairs = (long long)d.batch * d.heads_kv;
  if (G > 0) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, true, OUT_BF16>), dim3((unsigned)(pairs * A.nlt * A.nseg)), dim3(kThreads),
                       0, stream, A);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const long long per_seg = pairs * G * 2 * D;
    hipLaunchKernelGGL(bwd_lm_reduce_kernel, dim3((unsigned)((per_seg + 255) / 256)), dim3(256), 0, stream, part,
                       lmg, per_seg, lay.nseg);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, false, OUT_BF16>), dim3((unsigned)(pairs * A.nkt)), dim3(kThreads), 0,
                     stream, A);
  return hipGetLastError();
}

}  // namespace

// Workspace layout of the backward (all float32): LD [B*Hq][n_pad] (lse2, D)
// pairs, then the landmark partials [nseg][B*Hkv][G][2][D], then the summed
// landmark gradients [B*Hkv][G][2][D].  Each part starts on 256 bytes.
BwdLayout bwd_layout(const msa_attn_desc& d) {
  BwdLayout l;
  const int n = d.seq_len, G = d.num_landmarks;
  l.n_pad = (n + kPad - 1) / kPad * kPad;
  // segments of query rows for the landmark gradients: at least 1024 rows,
  // at most 128 segments (one workgroup per segment and landmark tile: small
  // enough that the unequal landmark work per segment balances over the CUs)
  int seg = (n + 127) / 128;
  seg = seg < 1024 ? 1024 : seg;
  seg = (seg + QB - 1) / QB * QB;
  l.seg = seg;
  l.nseg = G > 0 ? (n + seg - 1) / seg : 0;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t ld = (size_t)d.batch * d.heads_q * l.n_pad * 8;
  const size_t lm = (size_t)d.batch * d.heads_kv * G * 2 * d.head_dim * 4;
  l.ld_off = 0;
  l.part_off = up(ld);
  l.lmg_off = l.part_off + up((size_t)l.nseg * lm);
  l.bytes = l.lmg_off + up(lm);
  return l;
}

hipError_t launch_attn_bwd(const msa_attn_desc& d, const void* Q, const void* K, const void* V, const void* Kbar,
                           const void* Vbar, const void* O, const float* LSE, const void* dO, void* workspace,
                           void* dQ, void* dK, void* dV, hipStream_t stream) {
  const BwdLayout lay = bwd_layout(d);
  const bool ob = d.out_dtype == MSA_DTYPE_BF16;
  if (d.head_dim == 128) {
    return ob ? launch_bwd_t<128, true>(d, lay, Q, K, V, Kbar, Vbar, O, LSE, dO, workspace, dQ, dK, dV, stream)
              : launch_bwd_t<128, false>(d, lay, Q, K, V, Kbar, Vbar, O, LSE, dO, workspace, dQ, dK, dV, stream);
  }
  return ob ? launch_bwd_t<64, true>(d, lay, Q, K, V, Kbar, Vbar, O, LSE, dO, workspace, dQ, dK, dV, stream)
            : launch_bwd_t<64, false>(d, lay, Q, K, V, Kbar, Vbar, O, LSE, dO, workspace, dQ, dK, dV, stream);
}

}  // namespace msa
