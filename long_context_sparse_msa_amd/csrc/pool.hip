// Landmark pooling: Kbar[b,g,blk,:] = mean of K[b,g,blk*L .. blk*L+L-1,:]
// and the same for V (the landmark tokens of the page "Scaling GPU Cluster
// for Million Token Context", section "Why Sparse Attention Changes the
// Game", taken as block means).  Pure streaming: every input byte is read
// once with 16-byte loads; float32 accumulation in a fixed order, so the
// result is deterministic; round-to-nearest-even into the input dtype.
#include "msa_device.hpp"
#include "msa_internal.hpp"

namespace msa {
namespace {

template <typename T>
struct Chunk;  // one 16-byte load

template <>
struct Chunk<uint16_t> {
  static constexpr int kElems = 8;
  __device__ static void add(float* acc, const u32x4& v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += bf16_bits_to_f32(v[e] & 0xffffu);
      acc[2 * e + 1] += bf16_bits_to_f32(v[e] >> 16);
    }
  }
  __device__ static void store(uint16_t* dst, const float* vals) {
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(vals[2 * e], vals[2 * e + 1]);
    *reinterpret_cast<u32x4*>(dst) = o;
  }
};

template <>
struct Chunk<float> {
  static constexpr int kElems = 4;
  __device__ static void add(float* acc, const u32x4& v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += __uint_as_float(v[e]);
  }
  __device__ static void store(float* dst, const float* vals) {
    *reinterpret_cast<f32x4*>(dst) = f32x4{vals[0], vals[1], vals[2], vals[3]};
  }
};

// One workgroup per (tensor, batch*kv_head, landmark).  Threads are laid
// out as kRowLanes row lanes x kChunks 16-byte column chunks; row lane rl
// sums rows rl, rl + kRowLanes, ... of the block, then the row lanes are
// added in order through LDS.
template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ K, const T* __restrict__ V,
                                                   T* __restrict__ Kbar, T* __restrict__ Vbar, int n,
                                                   int G, int L, int blocks_per_tensor) {
  constexpr int kE = Chunk<T>::kElems;
  constexpr int kChunks = D / kE;
  constexpr int kRowLanes = 256 / kChunks;
  __shared__ float red[kRowLanes][D + 1];

  const int wg = blockIdx.x;
  const bool is_v = wg >= blocks_per_tensor;
  const int blk = is_v ? wg - blocks_per_tensor : wg;  // over batch*kv_heads*G
  const int bh = blk / G;
  const int lm = blk - bh * G;
  const T* src = (is_v ? V : K) + ((size_t)bh * n + (size_t)lm * L) * D;
  T* dst = (is_v ? Vbar : Kbar) + (size_t)blk * D;

  const int ch = threadIdx.x % kChunks;
  const int rl = threadIdx.x / kChunks;
  float acc[kE];
#pragma unroll
  for (int e = 0; e < kE; ++e) acc[e] = 0.f;

  const u32x4* p = reinterpret_cast<const u32x4*>(src) + ch;
  constexpr int kStride = kChunks;  // u32x4 per row
  int r = rl;
  for (; r + 3 * kRowLanes < L; r += 4 * kRowLanes) {
    const u32x4 a = p[(size_t)r * kStride];
    const u32x4 b = p[(size_t)(r + kRowLanes) * kStride];
    const u32x4 c = p[(size_t)(r + 2 * kRowLanes) * kStride];
    const u32x4 d = p[(size_t)(r + 3 * kRowLanes) * kStride];
    Chunk<T>::add(acc, a);
    Chunk<T>::add(acc, b);
    Chunk<T>::add(acc, c);
    Chunk<T>::add(acc, d);
  }
  for (; r < L; r += kRowLanes) Chunk<T>::add(acc, p[(size_t)r * kStride]);

#pragma unroll
  for (int e = 0; e < kE; ++e) red[rl][ch * kE + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < kChunks) {
    float out[kE];
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      float s = 0.f;
      for (int q = 0; q < kRowLanes; ++q) s += red[q][threadIdx.x * kE + e];
      out[e] = s / (float)L;
    }
    Chunk<T>::store(dst + threadIdx.x * kE, out);
  }
}

template <typename T, int D>
hipError_t launch_pool_t(const msa_attn_desc& d, const void* K, const void* V, void* Kb, void* Vb,
                         hipStream_t stream) {
  const int G = d.num_landmarks;
  const int L = d.seq_len / G;
  const int per = d.batch * d.heads_kv * G;
  hipLaunchKernelGGL((pool_kernel<T, D>), dim3(2 * per), dim3(256), 0, stream,
                     static_cast<const T*>(K), static_cast<const T*>(V), static_cast<T*>(Kb),
                     static_cast<T*>(Vb), d.seq_len, G, L, per);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pool(const msa_attn_desc& d, const void* K, const void* V, void* Kbar, void* Vbar,
                       hipStream_t stream) {
  if (d.in_dtype == MSA_DTYPE_BF16) {
    return d.head_dim == 128 ? launch_pool_t<uint16_t, 128>(d, K, V, Kbar, Vbar, stream)
                             : launch_pool_t<uint16_t, 64>(d, K, V, Kbar, Vbar, stream);
  }
  return d.head_dim == 128 ? launch_pool_t<float, 128>(d, K, V, Kbar, Vbar, stream)
                           : launch_pool_t<float, 64>(d, K, V, Kbar, Vbar, stream);
}

}  // namespace msa
