// Decode: one new query per sequence at position ctx-1 attends to its causal
// window of the KV cache plus the visible landmarks, split into chunks whose
// softmax statistics are merged afterwards (the single-GPU form of the
// Ring Attention aggregation on the page "Training at 1M+ Token Context:
// Ring Attention, YaRN, NTK-Aware Scaling GPU Cost", Ring Attention
// paragraph: partial results per KV block, combined through their softmax
// statistics, no score matrix kept).
//
// Pass 1 (decode_split_kernel): one workgroup per (sequence, KV head,
// chunk).  The query heads of the KV group (<= 16) are packed into the N
// dimension of v_mfma_f32_16x16x32_bf16, so each K/V row is read from HBM
// exactly once for all of them.  The four wavefronts take 32-entry blocks of
// the chunk round-robin; K fragments go straight from HBM into MFMA operand
// registers, V is transposed through a per-wave LDS slab.  Each wave keeps
// its own online softmax; the four are merged in LDS and the chunk's
// normalised output and natural-log LSE go to the workspace.
// Pass 2 (decode_merge_kernel): LSE-weighted sum of the chunk results.
#include "msa_device.hpp"
#include "msa_internal.hpp"
#include "msa_plan.hpp"

namespace msa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kBlk = 32;             // entries per wave step
constexpr int kVS = kBlk + 4;        // V^T slab row stride (elements)

__device__ __forceinline__ float max16(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float sum16(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

template <int D>
struct Slab {
  static constexpr int kStageBytes = kWaves * D * kVS * 2;
  static constexpr int kMergeBytes = kWaves * (2 * 16 + 16 * D) * 4;
  static constexpr int kBytes = kStageBytes > kMergeBytes ? kStageBytes : kMergeBytes;
};

template <int D>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ Kc, const uint16_t* __restrict__ Vc,
    const uint16_t* __restrict__ Kb, const uint16_t* __restrict__ Vb, float* __restrict__ ws_o,
    float* __restrict__ ws_lse, int B, int Hq, int Hkv, int ctx, int G, float scale_log2, int lm,
    int win0, int E, int chunk, int S) {
  constexpr int KK = D / 32;
  constexpr int MB = D / 16;
  constexpr int kVItems = (kBlk / 4) * (D / 8) / 64;  // (4-entry, 8-dim) items per lane
  __shared__ __align__(16) unsigned char smem[Slab<D>::kBytes];

  const int wg = blockIdx.x;
  const int c = wg % S;
  const int bk = wg / S;  // b * Hkv + kvh
  const int kvh = bk % Hkv;
  const int b = bk / Hkv;
  const int grp = Hq / Hkv;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c16 = lane & 15;
  const int g4 = lane >> 4;

  const int e0 = c * chunk;
  const int e1 = min(E, e0 + chunk);

  const uint16_t* kc = Kc + (size_t)bk * ctx * D;
  const uint16_t* vc = Vc + (size_t)bk * ctx * D;
  const uint16_t* kb = G > 0 ? Kb + (size_t)bk * G * D : kc;
  const uint16_t* vb = G > 0 ? Vb + (size_t)bk * G * D : vc;

  // Row address of entry e of the ordered list (landmarks, then window).
  auto krow = [&](int e) -> const uint16_t* {
    return e < lm ? kb + (size_t)e * D : kc + (size_t)(win0 + e - lm) * D;
  };
  auto vrow = [&](int e) -> const uint16_t* {
    return e < lm ? vb + (size_t)e * D : vc + (size_t)(win0 + e - lm) * D;
  };

  // query fragments: B[k = dim][n = head in group]
  bf16x8 qf[KK];
  {
    const int hh = c16 < grp ? c16 : 0;
    const uint16_t* qp = q + ((size_t)b * Hq + kvh * grp + hh) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (c16 < grp) v = *reinterpret_cast<const u32x4*>(qp + kk * 32 + g4 * 8);
      qf[kk] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x4 o[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) o[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -1e30f;
  float l = 0.f;

  uint16_t* slab = reinterpret_cast<uint16_t*>(smem) + wave * D * kVS;
  const int eg = lane % 8;  // V staging: entries eg*4 .. eg*4+3
  const int dg0 = lane / 8;

  for (int base = e0 + wave * kBlk; base < e1; base += kWaves * kBlk) {
    // ---- loads (invalid entries read a valid row and are masked)
    u32x4 kreg[2][KK];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      int e = base + kb2 * 16 + c16;
      e = e < e1 ? e : e1 - 1;
      const uint16_t* p = krow(e);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) kreg[kb2][kk] = *reinterpret_cast<const u32x4*>(p + kk * 32 + g4 * 8);
    }
    u32x4 vreg[kVItems][4];
#pragma unroll
    for (int it = 0; it < kVItems; ++it) {
      const int dg = dg0 + 8 * it;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int e = base + eg * 4 + r;
        e = e < e1 ? e : e1 - 1;
        vreg[it][r] = *reinterpret_cast<const u32x4*>(vrow(e) + dg * 8);
      }
    }

    // ---- V^T into this wave's slab
#pragma unroll
    for (int it = 0; it < kVItems; ++it) {
      const int dg = dg0 + 8 * it;
#pragma unroll
      for (int ee = 0; ee < 8; ++ee) {
        const int word = ee >> 1;
        const int sh = (ee & 1) * 16;
        u32x2 pk;
        pk[0] = ((vreg[it][0][word] >> sh) & 0xffffu) | (((vreg[it][1][word] >> sh) & 0xffffu) << 16);
        pk[1] = ((vreg[it][2][word] >> sh) & 0xffffu) | (((vreg[it][3][word] >> sh) & 0xffffu) << 16);
        *reinterpret_cast<u32x2*>(slab + (dg * 8 + ee) * kVS + eg * 4) = pk;
      }
    }

    // ---- S^T = K q^T: acc[kb2][i] = entry kb2*16 + g4*4 + i, head c16
    f32x4 acc[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      acc[kb2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        acc[kb2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kreg[kb2][kk]), qf[kk],
                                                           acc[kb2], 0, 0, 0);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = base + kb2 * 16 + g4 * 4 + i;
        const float s = e < e1 ? acc[kb2][i] * scale_log2 : -INFINITY;
        acc[kb2][i] = s;
        mx = fmaxf(mx, s);
      }
    }
    mx = max16(mx);
    const float m_new = fmaxf(m, mx);
    const float alpha = exp2f(m - m_new);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) o[mb] *= alpha;
    float p[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = exp2f(acc[0][i] - m);
      p[4 + i] = exp2f(acc[1][i] - m);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) l += p[i];
    u32x4 pk;
#pragma unroll
    for (int i = 0; i < 4; ++i) pk[i] = pack_bf16x2(p[2 * i], p[2 * i + 1]);
    const bf16x8 pf = __builtin_bit_cast(bf16x8, pk);

    __builtin_amdgcn_s_waitcnt(0xc07f);  // LDS writes of this wave are done
    __builtin_amdgcn_wave_barrier();
    // ---- O^T += V^T P^T
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const uint16_t* vr = slab + (mb * 16 + c16) * kVS + g4 * 4;
      const u32x2 lo = *reinterpret_cast<const u32x2*>(vr);
      const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + 16);
      const u32x4 vv = {lo[0], lo[1], hi[0], hi[1]};
      o[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vv), pf, o[mb], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- merge the four waves in LDS
  l = sum16(l);
  __syncthreads();  // slabs no longer needed
  float* mw = reinterpret_cast<float*>(smem);  // [4][16]
  float* lw = mw + kWaves * 16;                // [4][16]
  float* ow = lw + kWaves * 16;                // [4][16][D]
  if (g4 == 0) {
    mw[wave * 16 + c16] = m;
    lw[wave * 16 + c16] = l;
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ow[(wave * 16 + c16) * D + mb * 16 + g4 * 4 + i] = o[mb][i];
  }
  __syncthreads();

  for (int idx = tid; idx < grp * D; idx += kThreads) {
    const int hh = idx / D;
    const int d = idx % D;
    float M = -1e30f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) M = fmaxf(M, mw[v * 16 + hh]);
    float num = 0.f;
    float den = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      const float a = exp2f(mw[v * 16 + hh] - M);
      num += a * ow[(v * 16 + hh) * D + d];
      den += a * lw[v * 16 + hh];
    }
    const size_t slot = ((size_t)c * B + b) * Hq + kvh * grp + hh;
    ws_o[slot * D + d] = den > 0.f ? num / den : 0.f;
    if (d == 0) ws_lse[slot] = den > 0.f ? (M + log2f(den)) * kLn2 : -INFINITY;
  }
}

// One wavefront per (sequence, query head).
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
  for (int c = 0; c < S; ++c) M = fmaxf(M, ws_lse[(size_t)c * BH + bh]);
  float acc[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) acc[e] = 0.f;
  float tot = 0.f;
  for (int c = 0; c < S; ++c) {
    const float lc = ws_lse[(size_t)c * BH + bh];
    if (lc == -INFINITY) continue;  // empty chunk
    const float wgt = exp2f((lc - M) * kLog2e);
    tot += wgt;
    const float* oc = ws_o + ((size_t)c * BH + bh) * D;
#pragma unroll
    for (int e = 0; e < kPer; ++e) acc[e] = fmaf(wgt, oc[lane + 64 * e], acc[e]);
  }
  const float inv = 1.0f / tot;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const float v = acc[e] * inv;
    if constexpr (OUT_BF16) {
      static_cast<uint16_t*>(Out)[(size_t)bh * D + lane + 64 * e] = f32_to_bf16_bits(v);
    } else {
      static_cast<float*>(Out)[(size_t)bh * D + lane + 64 * e] = v;
    }
  }
  if (LSE != nullptr && lane == 0) LSE[bh] = M + logf(tot);
}

template <int D>
hipError_t launch_t(const msa_decode_desc& d, const void* q, const void* Kc, const void* Vc,
                    const void* Kb, const void* Vb, float* ws_o, float* ws_lse, void* O, float* LSE,
                    hipStream_t stream) {
  const DecodePlan p = decode_plan(d.ctx_len, d.window, d.num_landmarks, d.num_splits);
  const long long wgs = (long long)d.batch * d.heads_kv * d.num_splits;
  hipLaunchKernelGGL((decode_split_kernel<D>), dim3((unsigned)wgs), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(Kc),
                     static_cast<const uint16_t*>(Vc), static_cast<const uint16_t*>(Kb),
                     static_cast<const uint16_t*>(Vb), ws_o, ws_lse, d.batch, d.heads_q, d.heads_kv,
                     d.ctx_len, d.num_landmarks, d.scale * kLog2e, p.lm, p.win0, p.entries, p.chunk,
                     d.num_splits);
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
                         const void* Kbar, const void* Vbar, float* ws_o, float* ws_lse, void* O,
                         float* LSE, hipStream_t stream) {
  return d.head_dim == 128 ? launch_t<128>(d, q, Kc, Vc, Kbar, Vbar, ws_o, ws_lse, O, LSE, stream)
                           : launch_t<64>(d, q, Kc, Vc, Kbar, Vbar, ws_o, ws_lse, O, LSE, stream);
}

}  // namespace msa
