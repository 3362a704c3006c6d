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
//  * A workgroup owns BM = 128 query rows of one head (4 wavefronts x 32
//    rows) and walks only the key tiles that matter: the landmark tiles
//    0 .. ceil(c(r_last)/64)-1, then the window tiles covering
//    [r_first-w+1, r_last] (closed forms in msa_plan.hpp).  Masks are
//    evaluated only on edge tiles.
//  * Both contractions run on v_mfma_f32_16x16x32_bf16.  Scores are formed
//    transposed, S^T = K Q^T, so that each lane's accumulator holds 16 keys
//    of one query row -- exactly the B operand layout of O^T = V^T P^T.  P
//    therefore never leaves registers, the row max/sum need only two
//    cross-lane steps, and the per-row rescale of O is a per-lane scalar.
//  * K tiles are staged row-major and V tiles transposed in LDS (padded
//    strides keep both the staging writes and the operand reads free of
//    bank conflicts), double-buffered with one barrier per tile; the next
//    tile's global loads are in flight while the current one is computed.
//  * The online softmax works in base 2 with scale*log2(e) folded into the
//    fp32 scores.
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

template <int D>
struct Lds {
  static constexpr int KS = D + 8;   // K row stride (elements): 16-byte pad
  static constexpr int VS = BN + 4;  // V^T row stride (elements): 8-byte pad
  static constexpr int kTile = BN * KS;
  static constexpr int vTile = D * VS;
  static constexpr int kBuf = kTile + vTile;  // one buffer (elements)
};

// Global -> register staging of one K/V tile (64 keys x D).
template <int D>
struct TileLoader {
  static constexpr int kChunksK = BN * D / 8 / kThreads;      // 16-byte chunks of K per thread
  static constexpr int kVItems = 16 * (D / 8);                 // (4-key group, 8-dim group) items
  u32x4 kreg[kChunksK];
  u32x4 vreg[4];

  // rows [row0, row0+64) of src (clamped to valid-1; clamped rows are masked)
  __device__ void load(const uint16_t* __restrict__ Ksrc, const uint16_t* __restrict__ Vsrc,
                       int row0, int valid, int tid) {
#pragma unroll
    for (int c = 0; c < kChunksK; ++c) {
      const int idx = tid + c * kThreads;
      const int r = idx / (D / 8);
      const int col = idx % (D / 8);
      int row = row0 + r;
      row = row < valid ? row : valid - 1;
      kreg[c] = *reinterpret_cast<const u32x4*>(Ksrc + (size_t)row * D + col * 8);
    }
    if (tid < kVItems) {
      const int kg = tid % 16;
      const int dg = tid / 16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int row = row0 + kg * 4 + r;
        row = row < valid ? row : valid - 1;
        vreg[r] = *reinterpret_cast<const u32x4*>(Vsrc + (size_t)row * D + dg * 8);
      }
    }
  }

  __device__ void store(uint16_t* __restrict__ buf, int tid) const {
    using L = Lds<D>;
#pragma unroll
    for (int c = 0; c < kChunksK; ++c) {
      const int idx = tid + c * kThreads;
      const int r = idx / (D / 8);
      const int col = idx % (D / 8);
      *reinterpret_cast<u32x4*>(buf + r * L::KS + col * 8) = kreg[c];
    }
    if (tid < kVItems) {
      const int kg = tid % 16;
      const int dg = tid / 16;
      uint16_t* vt = buf + L::kTile;
      // 4 keys x 8 dims in registers -> 8 rows of V^T, 4 keys each.
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int word = e >> 1;
        const int sh = (e & 1) * 16;
        const uint32_t a = (vreg[0][word] >> sh) & 0xffffu;
        const uint32_t b = (vreg[1][word] >> sh) & 0xffffu;
        const uint32_t c = (vreg[2][word] >> sh) & 0xffffu;
        const uint32_t d = (vreg[3][word] >> sh) & 0xffffu;
        u32x2 pk;
        pk[0] = a | (b << 16);
        pk[1] = c | (d << 16);
        *reinterpret_cast<u32x2*>(vt + (dg * 8 + e) * L::VS + kg * 4) = pk;
      }
    }
  }
};

__device__ __forceinline__ float wave_max16(float x) {
  // max over the 4 lanes that share (lane mod 16)
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float wave_sum16(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ Kb, const uint16_t* __restrict__ Vb, void* __restrict__ Out,
    float* __restrict__ LSE, int Hq, int Hkv, int n, int w, int G, int L, float scale_log2, int T) {
  using LD = Lds<D>;
  constexpr int KK = D / 32;  // k-steps of the QK^T contraction
  constexpr int MB = D / 16;  // 16-dim blocks of O^T
  __shared__ __align__(16) uint16_t lds[2 * LD::kBuf];

  // ---- which (batch, head, query tile) this workgroup owns
  const int j = xcd_remap(blockIdx.x, gridDim.x);
  const int grp = Hq / Hkv;
  const int h_in = j % grp;
  int rest = j / grp;
  const int t = T - 1 - rest % T;  // heaviest tiles first
  rest /= T;
  const int kvh = rest % Hkv;
  const int b = rest / Hkv;
  const int h = kvh * grp + h_in;

  const TileRange tr = tile_range(t, BM, BN, n, w, G, L);
  const int n_win = tr.kt_hi - tr.kt_lo + 1;
  const int n_tiles = tr.n_lm_tiles + n_win;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c16 = lane & 15;
  const int g4 = lane >> 4;

  const size_t kv_off = ((size_t)b * Hkv + kvh) * (size_t)n * D;
  const size_t lm_off = ((size_t)b * Hkv + kvh) * (size_t)(G > 0 ? G : 1) * D;
  const size_t q_off = ((size_t)b * Hq + h) * (size_t)n * D;
  const uint16_t* Kw = K + kv_off;
  const uint16_t* Vw = V + kv_off;
  const uint16_t* Kl = G > 0 ? Kb + lm_off : Kw;
  const uint16_t* Vl = G > 0 ? Vb + lm_off : Vw;

  // ---- this wave's rows and its own sub-range of the tile list
  const int wr0 = tr.r0 + wave * 32;
  const int wr1 = min(wr0 + 31, n - 1);
  const bool wave_live = wr0 <= n - 1;
  int row[2];
  int lmc[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    row[nb] = wr0 + nb * 16 + c16;
    lmc[nb] = lm_count(row[nb], w, G, L);
  }
  const int wlm_lo = lm_count(wr0, w, G, L);
  const int wlm_hi = wave_live ? lm_count(wr1, w, G, L) : 0;

  // ---- Q fragments (B operand of S^T = K Q^T), held for the whole tile walk
  bf16x8 qf[2][KK];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row[nb] < n) v = *reinterpret_cast<const u32x4*>(Q + q_off + (size_t)row[nb] * D + kk * 32 + g4 * 8);
      qf[nb][kk] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x4 o[MB][2];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    o[mb][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    o[mb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float m[2] = {-1e30f, -1e30f};  // running max, base-2 scaled units
  float l[2] = {0.f, 0.f};        // this lane's share of the running sum

  TileLoader<D> ld;
  auto issue = [&](int it) {
    if (it < tr.n_lm_tiles) {
      ld.load(Kl, Vl, it * BN, G, tid);
    } else {
      ld.load(Kw, Vw, (tr.kt_lo + it - tr.n_lm_tiles) * BN, n, tid);
    }
  };

  issue(0);
  ld.store(lds, tid);
  __syncthreads();

  for (int it = 0; it < n_tiles; ++it) {
    const bool more = it + 1 < n_tiles;
    if (more) issue(it + 1);

    const uint16_t* kt = lds + (it & 1) * LD::kBuf;
    const uint16_t* vt = kt + LD::kTile;
    const bool is_lm = it < tr.n_lm_tiles;
    const int key0 = is_lm ? it * BN : (tr.kt_lo + it - tr.n_lm_tiles) * BN;

    // Does this wave see anything in the tile, and without a mask?
    bool any, interior;
    if (is_lm) {
      any = wave_live && key0 < wlm_hi;
      interior = (key0 + BN) <= wlm_lo;
    } else {
      any = wave_live && key0 <= wr1 && key0 + BN - 1 >= wr0 - w + 1;
      interior = key0 + BN - 1 <= wr0 && key0 >= wr1 - w + 1;
    }

    if (any) {
      // ---- S^T = K Q^T : acc[kb][nb] holds keys kb*16 + g4*4 + (0..3) of row nb*16 + c16
      f32x4 acc[4][2];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        acc[kb][0] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc[kb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const bf16x8 kf =
              *reinterpret_cast<const bf16x8*>(kt + (kb * 16 + c16) * LD::KS + kk * 32 + g4 * 8);
          acc[kb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[0][kk], acc[kb][0], 0, 0, 0);
          acc[kb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[1][kk], acc[kb][1], 0, 0, 0);
        }
      }

      // ---- scale into base-2 units, mask edge tiles
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float s = acc[kb][nb][i] * scale_log2;
            if (!interior) {
              const int key = key0 + kb * 16 + g4 * 4 + i;
              const bool vis = is_lm ? (key < lmc[nb]) : (key <= row[nb] && key > row[nb] - w);
              s = vis ? s : -INFINITY;
            }
            acc[kb][nb][i] = s;
          }
        }
      }

      // ---- online softmax
      float alpha[2];
      bool rescale = false;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          mx = fmaxf(mx, fmaxf(fmaxf(acc[kb][nb][0], acc[kb][nb][1]), fmaxf(acc[kb][nb][2], acc[kb][nb][3])));
        }
        mx = wave_max16(mx);
        const float m_new = fmaxf(m[nb], mx);
        alpha[nb] = exp2f(m[nb] - m_new);
        rescale |= m_new > m[nb];
        m[nb] = m_new;
      }
      if (__any(rescale)) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          l[nb] *= alpha[nb];
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) o[mb][nb] *= alpha[nb];
        }
      }

      // P = exp2(s - m), packed to bf16 as the B operand of O^T += V^T P^T.
      bf16x8 pf[2][2];  // [kb2][nb]
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        float rs = 0.f;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          float p[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p[i] = exp2f(acc[2 * kb2][nb][i] - m[nb]);
            p[4 + i] = exp2f(acc[2 * kb2 + 1][nb][i] - m[nb]);
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) rs += p[i];
          u32x4 pk;
#pragma unroll
          for (int i = 0; i < 4; ++i) pk[i] = pack_bf16x2(p[2 * i], p[2 * i + 1]);
          pf[kb2][nb] = __builtin_bit_cast(bf16x8, pk);
        }
        l[nb] += rs;
      }

      // ---- O^T += V^T P^T
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const uint16_t* vrow = vt + (mb * 16 + c16) * LD::VS + kb2 * 32 + g4 * 4;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 16);
          const u32x4 vv = {lo[0], lo[1], hi[0], hi[1]};
          const bf16x8 vf = __builtin_bit_cast(bf16x8, vv);
          o[mb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[kb2][0], o[mb][0], 0, 0, 0);
          o[mb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[kb2][1], o[mb][1], 0, 0, 0);
        }
      }
    }

    if (more) ld.store(lds + ((it + 1) & 1) * LD::kBuf, tid);
    __syncthreads();
  }

  // ---- epilogue: O = O_acc / l, LSE = (m + log2 l) ln 2
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float lt = wave_sum16(l[nb]);
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    if (row[nb] < n) {
      const size_t base = q_off + (size_t)row[nb] * D;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int dcol = mb * 16 + g4 * 4;
        const f32x4 v = o[mb][nb] * inv;
        if constexpr (OUT_BF16) {
          u32x2 pk;
          pk[0] = pack_bf16x2(v[0], v[1]);
          pk[1] = pack_bf16x2(v[2], v[3]);
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(Out) + base + dcol) = pk;
        } else {
          *reinterpret_cast<f32x4*>(static_cast<float*>(Out) + base + dcol) = v;
        }
      }
      if (LSE != nullptr && g4 == 0) {
        LSE[((size_t)b * Hq + h) * n + row[nb]] = (m[nb] + log2f(lt)) * kLn2;
      }
    }
  }
}

template <int D, bool OUT_BF16>
hipError_t launch_t(const msa_attn_desc& d, const void* Q, const void* K, const void* V,
                    const void* Kb, const void* Vb, void* O, float* LSE, hipStream_t stream) {
  const int n = d.seq_len;
  const int T = (n + BM - 1) / BM;
  const int G = d.num_landmarks;
  const int L = G > 0 ? n / G : 1;
  const long long wgs = (long long)d.batch * d.heads_q * T;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, OUT_BF16>), dim3((unsigned)wgs), dim3(kThreads), 0,
                     stream, static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K),
                     static_cast<const uint16_t*>(V), static_cast<const uint16_t*>(Kb),
                     static_cast<const uint16_t*>(Vb), O, LSE, d.heads_q, d.heads_kv, n, d.window, G, L,
                     d.scale * kLog2e, T);
  return hipGetLastError();
}

}  // namespace

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
