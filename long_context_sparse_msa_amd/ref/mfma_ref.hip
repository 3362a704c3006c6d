// Measured references for bench.py (not part of libmsa's interface): the
// matrix-core throughput of two fixed instruction streams on this GPU, so
// that the prefill kernel's rate can be set against what the hardware
// delivers for the same kind of work on the same box.
//
//  mode 0  32x32x16 bf16 MFMAs on register operands, four independent
//          accumulators: the matrix cores' ceiling under this part's clock
//          and power behaviour for random bf16 data.
//  mode 1  the prefill's per-tile dependency chain with its LDS operand
//          traffic and no HBM traffic: per trip, QK (16 MFMAs, A operands by
//          ds_read_b128 from a swizzled 64 x 128 tile) -> for each of the 32
//          scores a lane holds, exp2 of an FMA and a sum, 16 bf16 packs and
//          16 bf16 dot products (all depending on QK) -> PV (16 MFMAs, A
//          operands by pairs of ds_read_b64_tr_b16, B the packed P), two
//          wavefronts per SIMD (64 KB of LDS per workgroup).
//
// Both run 2048 workgroups of 256 threads; every LDS offset lies inside the
// first 32 KB of the workgroup's array (checked on the host before launch).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;

constexpr int kRB = 256;            // bytes per 128-dim bf16 row
constexpr int kCH = 16;             // 16-byte chunks per row
constexpr int kTile = 64 * kRB;     // one 64-row tile
constexpr int kLdsBytes = 4 * kTile;
constexpr int kBlocks = 2048;
constexpr int kThreads = 256;
constexpr int kInWords = 4096 * 4;  // random bf16 pairs the kernels read

// K-operand read of step (ks, mb): row mb*32 + lane%32, chunk (2ks + lane/32) ^ (row % 16).
__host__ __device__ inline uint32_t k_off(int lane, int ks, int mb) {
  const int r32 = lane & 31, c = ks * 2 + (lane >> 5);
  return (uint32_t)((mb * 32 + r32) * kRB + ((c ^ (r32 % kCH)) * 16));
}
// V^T-operand transpose read of step (kk, db) in the second tile: key kk*16 + (g/2)*4 + j/4,
// dims db*32 + (g%2)*16 + 4*(j%4), chunk swizzled by 4*(key % 4).
__host__ __device__ inline uint32_t v_off(int lane, int db, int kk) {
  const int g = lane >> 4, j = lane & 15;
  const int key = kk * 16 + (g >> 1) * 4 + (j >> 2);
  const int d = db * 32 + (g & 1) * 16 + 4 * (j & 3);
  return (uint32_t)(kTile + key * kRB + (((d / 8) ^ ((key % 4) * (kCH / 4))) * 16) + (d % 8) * 2);
}

__device__ inline void fill_lds(unsigned char* smem, const uint32_t* in) {
  for (int i = threadIdx.x; i < 2 * kTile / 16; i += kThreads)
    reinterpret_cast<u32x4*>(smem)[i] = reinterpret_cast<const u32x4*>(in)[(blockIdx.x * 7 + i) % (kInWords / 4)];
  __syncthreads();
}

__global__ __launch_bounds__(kThreads, 2) void mfma_register_kernel(const uint32_t* __restrict__ in,
                                                                    float* __restrict__ out, int iters) {
  __shared__ __align__(16) unsigned char smem[kLdsBytes];  // holds occupancy at two workgroups per CU
  fill_lds(smem, in);
  const int tid = threadIdx.x;
  const u32x4 b0 = reinterpret_cast<const u32x4*>(in)[(blockIdx.x * kThreads + tid) % (kInWords / 4)];
  const u32x4 b1 = reinterpret_cast<const u32x4*>(in)[(blockIdx.x * kThreads + tid + 1) % (kInWords / 4)];
  const bf16x8 B0 = __builtin_bit_cast(bf16x8, b0), B1 = __builtin_bit_cast(bf16x8, b1);
  f32x16 acc[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 32; ++m)
      acc[m % 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16((m & 1) ? B1 : B0, (m & 2) ? B1 : B0, acc[m % 4], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += acc[0][i] + acc[1][i] + acc[2][i] + acc[3][i];
  out[blockIdx.x * kThreads + tid] = s + (float)smem[tid];
}

__global__ __launch_bounds__(kThreads, 2) void mfma_chain_kernel(const uint32_t* __restrict__ in,
                                                                 float* __restrict__ out, int iters) {
  __shared__ __align__(16) unsigned char smem[kLdsBytes];
  fill_lds(smem, in);
  const int tid = threadIdx.x, lane = tid & 63;
  bf16x8 qf[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
    qf[k] = __builtin_bit_cast(bf16x8, reinterpret_cast<const u32x4*>(in)[(blockIdx.x * kThreads + tid + k) % (kInWords / 4)]);
  f32x16 o[4] = {};
  float l = 0.f, ls = 0.f;
  const float c2 = 0.1275f, nm = -4.0f;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  for (int it = 0; it < iters; ++it) {
    asm volatile("" ::: "memory");  // the operand reads stay inside the loop
    f32x16 s[2] = {};
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(smem + k_off(lane, m / 2, m % 2));
      s[m % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[m / 2], s[m % 2], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    float p[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e / 16][e % 16], c2, nm));
    float t = 0.f;
#pragma unroll
    for (int e = 0; e < 32; e += 2) t += p[e] + p[e + 1];
    ls += t;
    uint32_t w[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      w[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{p[2 * k], p[2 * k + 1]}, bf16x2));
      l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[k]), ones, l, false);
    }
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const uint32_t off = v_off(lane, m % 4, m / 4);
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(smem + off));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(smem + off + 8 * kRB));
      const u32x2 x = __builtin_bit_cast(u32x2, lo), y = __builtin_bit_cast(u32x2, hi);
      const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{x[0], x[1], y[0], y[1]});
      const int kk = m / 4;
      const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{w[kk * 4], w[kk * 4 + 1], w[kk * 4 + 2], w[kk * 4 + 3]});
      o[m % 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, o[m % 4], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  float r = l + ls;
#pragma unroll
  for (int i = 0; i < 16; ++i) r += o[0][i] + o[1][i] + o[2][i] + o[3][i];
  out[blockIdx.x * kThreads + tid] = r;
}

bool offsets_in_range() {
  for (int lane = 0; lane < 64; ++lane) {
    for (int m = 0; m < 16; ++m) {
      if (k_off(lane, m / 2, m % 2) + 16 > (uint32_t)(2 * kTile)) return false;
      if (v_off(lane, m % 4, m / 4) + 8 * kRB + 8 > (uint32_t)(2 * kTile)) return false;
    }
  }
  return true;
}

}  // namespace

// mode 0 or 1 (above); iters trips per launch (>= 1); the best of reps
// (>= 1) launches after one untimed launch.  Writes the best launch's
// milliseconds and the MFMA FLOPs one launch executes.  Returns 0, or a
// HIP error code (an invalid argument for a bad mode, iters or reps).
extern "C" int msa_ref_mfma(int mode, int iters, int reps, double* ms_out, double* flops_out) {
  if ((mode != 0 && mode != 1) || iters < 1 || reps < 1 || ms_out == nullptr || flops_out == nullptr ||
      !offsets_in_range())
    return (int)hipErrorInvalidValue;
  std::vector<uint32_t> h(kInWords);
  uint32_t x = 12345u;
  for (auto& e : h) {  // random bf16 pairs: random sign and mantissa, exponent near 1
    x = x * 1664525u + 1013904223u;
    const uint32_t lo = 0x3f00u | ((x >> 8) & 0x00ffu) | ((x & 1u) << 15);
    x = x * 1664525u + 1013904223u;
    const uint32_t hi = 0x3f00u | ((x >> 8) & 0x00ffu) | ((x & 1u) << 15);
    e = lo | (hi << 16);
  }
  uint32_t* din = nullptr;
  float* dout = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t err = hipMalloc(&din, h.size() * sizeof(uint32_t));
  if (err == hipSuccess) err = hipMalloc(&dout, (size_t)kBlocks * kThreads * sizeof(float));
  if (err == hipSuccess) err = hipMemcpy(din, h.data(), h.size() * sizeof(uint32_t), hipMemcpyHostToDevice);
  if (err == hipSuccess) err = hipEventCreate(&e0);
  if (err == hipSuccess) err = hipEventCreate(&e1);
  double best = 1e30;
  for (int r = -1; err == hipSuccess && r < reps; ++r) {
    err = hipEventRecord(e0, nullptr);
    if (err != hipSuccess) break;
    if (mode == 0)
      hipLaunchKernelGGL(mfma_register_kernel, dim3(kBlocks), dim3(kThreads), 0, nullptr, din, dout, iters);
    else
      hipLaunchKernelGGL(mfma_chain_kernel, dim3(kBlocks), dim3(kThreads), 0, nullptr, din, dout, iters);
    err = hipGetLastError();
    if (err == hipSuccess) err = hipEventRecord(e1, nullptr);
    if (err == hipSuccess) err = hipEventSynchronize(e1);
    float ms = 0.f;
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, e0, e1);
    if (err == hipSuccess && r >= 0 && ms < best) best = ms;
  }
  if (e0 != nullptr) (void)hipEventDestroy(e0);
  if (e1 != nullptr) (void)hipEventDestroy(e1);
  if (din != nullptr) (void)hipFree(din);
  if (dout != nullptr) (void)hipFree(dout);
  if (err != hipSuccess) return (int)err;
  *ms_out = best;
  *flops_out = 32.0 * 32768.0 * (double)iters * (double)kBlocks * 4.0;  // 32 MFMAs per trip per wavefront
  return 0;
}
