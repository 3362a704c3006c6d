// Sparse-attention prefill for float32 inputs (same operation as the bf16
// kernel, see attn_bf16.hip; this path serves full-precision problems such as
// small checking workloads).  fp32 all the way: dot products on the vector
// ALUs, K/V tiles staged in LDS, an online softmax per key.
//
// A workgroup owns 64 query rows of one head; each row is handled by 4
// lanes that split the head dimension, so a score is a 4-lane reduction.
// Only the landmark and window tiles listed by msa_plan.hpp are visited.
#include "msa_device.hpp"
#include "msa_internal.hpp"
#include "msa_plan.hpp"

namespace msa {
namespace {

constexpr int BM = kBM_F32;  // 64
constexpr int BN = kBN_F32;  // 64
constexpr int kThreads = 256;

template <int D>
__global__ __launch_bounds__(kThreads) void attn_fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ Kb, const float* __restrict__ Vb, float* __restrict__ Out,
    float* __restrict__ LSE, int Hq, int Hkv, int n, int w, int G, int L, float scale_log2, int T) {
  constexpr int DS = D / 4;  // dims per lane
  __shared__ __align__(16) float ks[BN][D];
  __shared__ __align__(16) float vs[BN][D];

  const int j = xcd_remap(blockIdx.x, gridDim.x);
  const int grp = Hq / Hkv;
  const int h_in = j % grp;
  int rest = j / grp;
  const int t = T - 1 - rest % T;
  rest /= T;
  const int kvh = rest % Hkv;
  const int b = rest / Hkv;
  const int h = kvh * grp + h_in;

  const TileRange tr = tile_range(t, BM, BN, n, w, G, L);
  const int n_tiles = tr.n_lm_tiles + (tr.kt_hi - tr.kt_lo + 1);

  const int tid = threadIdx.x;
  const int part = tid & 3;
  const int row = tr.r0 + (tid >> 2);
  const bool live = row < n;
  const int lmc = lm_count(row, w, G, L);

  const size_t kv_off = ((size_t)b * Hkv + kvh) * (size_t)n * D;
  const size_t lm_off = ((size_t)b * Hkv + kvh) * (size_t)(G > 0 ? G : 1) * D;
  const size_t q_off = ((size_t)b * Hq + h) * (size_t)n * D;

  float q[DS];
  float o[DS];
#pragma unroll
  for (int e = 0; e < DS; ++e) {
    q[e] = live ? Q[q_off + (size_t)row * D + part * DS + e] : 0.f;
    o[e] = 0.f;
  }
  float m = -1e30f;
  float l = 0.f;

  for (int it = 0; it < n_tiles; ++it) {
    const bool is_lm = it < tr.n_lm_tiles;
    const int key0 = is_lm ? it * BN : (tr.kt_lo + it - tr.n_lm_tiles) * BN;
    const float* ksrc = is_lm ? Kb + lm_off : K + kv_off;
    const float* vsrc = is_lm ? Vb + lm_off : V + kv_off;
    const int valid = is_lm ? G : n;

    __syncthreads();  // previous tile fully consumed
    for (int idx = tid; idx < BN * D / 4; idx += kThreads) {
      const int r = idx / (D / 4);
      const int c = idx % (D / 4);
      int src_row = key0 + r;
      src_row = src_row < valid ? src_row : valid - 1;
      reinterpret_cast<f32x4*>(&ks[r][0])[c] = reinterpret_cast<const f32x4*>(ksrc + (size_t)src_row * D)[c];
      reinterpret_cast<f32x4*>(&vs[r][0])[c] = reinterpret_cast<const f32x4*>(vsrc + (size_t)src_row * D)[c];
    }
    __syncthreads();

    for (int kk = 0; kk < BN; ++kk) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < DS; ++e) dot = fmaf(q[e], ks[kk][part * DS + e], dot);
      dot += __shfl_xor(dot, 1);
      dot += __shfl_xor(dot, 2);
      const int key = key0 + kk;
      const bool vis = is_lm ? (key < lmc) : (key <= row && key > row - w);
      if (vis) {
        const float s = dot * scale_log2;
        if (s > m) {
          const float alpha = exp2f(m - s);
          l *= alpha;
#pragma unroll
          for (int e = 0; e < DS; ++e) o[e] *= alpha;
          m = s;
        }
        const float p = exp2f(s - m);
        l += p;
#pragma unroll
        for (int e = 0; e < DS; ++e) o[e] = fmaf(p, vs[kk][part * DS + e], o[e]);
      }
    }
  }

  if (live) {
    const float inv = 1.0f / l;
#pragma unroll
    for (int e = 0; e < DS; ++e) Out[q_off + (size_t)row * D + part * DS + e] = o[e] * inv;
    if (LSE != nullptr && part == 0) LSE[((size_t)b * Hq + h) * n + row] = (m + log2f(l)) * kLn2;
  }
}

template <int D>
hipError_t launch_t(const msa_attn_desc& d, const void* Q, const void* K, const void* V,
                    const void* Kb, const void* Vb, void* O, float* LSE, hipStream_t stream) {
  const int n = d.seq_len;
  const int T = (n + BM - 1) / BM;
  const int G = d.num_landmarks;
  const int L = G > 0 ? n / G : 1;
  const long long wgs = (long long)d.batch * d.heads_q * T;
  hipLaunchKernelGGL((attn_fwd_f32_kernel<D>), dim3((unsigned)wgs), dim3(kThreads), 0, stream,
                     static_cast<const float*>(Q), static_cast<const float*>(K),
                     static_cast<const float*>(V), static_cast<const float*>(Kb),
                     static_cast<const float*>(Vb), static_cast<float*>(O), LSE, d.heads_q, d.heads_kv,
                     n, d.window, G, L, d.scale * kLog2e, T);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(const msa_attn_desc& d, const void* Q, const void* K, const void* V,
                           const void* Kbar, const void* Vbar, void* O, float* LSE,
                           hipStream_t stream) {
  return d.head_dim == 128 ? launch_t<128>(d, Q, K, V, Kbar, Vbar, O, LSE, stream)
                           : launch_t<64>(d, Q, K, V, Kbar, Vbar, O, LSE, stream);
}

}  // namespace msa
