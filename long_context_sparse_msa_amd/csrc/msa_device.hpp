// Device-side helpers shared by the gfx950 kernels: vector types for MFMA
// operands, bf16 <-> f32 conversion and the XCD-aware workgroup remap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even float -> bf16 bits (gfx950 has a native convert).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

// Two floats -> packed bf16 pair (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// Raw buffer resource over `bytes` bytes at `base` (stride 0, 32-bit data
// format): loads through it are range-checked, out-of-range ones return 0
// (or, for loads into LDS, write nothing).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Two floats -> packed bf16 pair with the native convert (RNE).
__device__ __forceinline__ uint32_t cvt_pk(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Stores one wavefront's 32 rows x D of results as bf16.  The values sit in
// the C layout of 32x32 MFMA accumulators of a transposed product: lane l
// holds row l%32, dims db*32 + jj*8 + (l/32)*4 + i in acc[db][jj*4+i].  Each
// is multiplied by `mul` (per lane), staged in `stage` (this wavefront's
// 32*(2D+16) bytes of LDS) and written so that every store instruction covers
// whole 128-byte lines, with the non-temporal hint: results written once need
// no place in the L2.  Rows at or past `nrows` are not written.  Every thread
// of the workgroup must call it, after the last read of the LDS it reuses.
template <int D>
__device__ __forceinline__ void store_rows_bf16_nt(const f32x16* acc, float mul, unsigned char* stage, int lane,
                                                   uint16_t* dst_row0, int nrows) {
  constexpr int RS = D * 2 + 16;  // staged row stride: 16-byte aligned, rows r and r+16 share banks
  const int r32 = lane & 31;
  const int g2 = lane >> 5;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int dcol = db * 32 + jj * 8 + g2 * 4;
      const u32x2 pk = {cvt_pk(acc[db][jj * 4 + 0] * mul, acc[db][jj * 4 + 1] * mul),
                        cvt_pk(acc[db][jj * 4 + 2] * mul, acc[db][jj * 4 + 3] * mul)};
      *reinterpret_cast<u32x2*>(stage + r32 * RS + dcol * 2) = pk;
    }
  }
  __syncthreads();
  constexpr int LPR = D * 2 / 16;  // lanes per row, 16 bytes each
  constexpr int RPI = 64 / LPR;    // rows per store instruction
#pragma unroll
  for (int k = 0; k < 32 / RPI; ++k) {
    const int rr = k * RPI + lane / LPR;
    const u32x4 v = *reinterpret_cast<const u32x4*>(stage + rr * RS + (lane % LPR) * 16);
    if (rr < nrows) {
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst_row0 + (size_t)rr * D + (lane % LPR) * 8));
    }
  }
}

// (x[l], x[l^32]) for every lane l, as a pair whose max or sum is the
// value over both halves of the wavefront.
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ds_read_b64_tr_b16 written as inline assembly.  For the builtin form the
// compiler assumes the read may alias any direct-to-LDS buffer load still in
// flight and puts a vmcnt(0) wait in front of it, which would stall every
// tile on the prefetch of the next one.  The caller orders the read after
// the loads of its own tile (wait + barrier) and waits for the result with
// lds_wait() before using it.  `addr` is the LDS byte address.
template <int OFF>
__device__ __forceinline__ u32x2 ds_read_tr16_b64(uint32_t addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
}

// Wait until at most n LDS operations are outstanding (n a constant after
// unrolling, 0..15).  LDS operations complete in issue order, so with n =
// the number of LDS reads issued after the ones that produced x (and y),
// their results are ready afterwards.  The values are tied to the wait:
// every use of them, including any copy, comes after it.  Build operands
// from the tied values only after this call.  x and y must be distinct
// objects (the same object twice makes the compiler copy it before the wait).
#define MSA_LGKM_SWITCH(n, ...)                                                          \
  switch (n) {                                                                         \
    case 0: asm volatile("s_waitcnt lgkmcnt(0)" : __VA_ARGS__); break;                 \
    case 1: asm volatile("s_waitcnt lgkmcnt(1)" : __VA_ARGS__); break;                 \
    case 2: asm volatile("s_waitcnt lgkmcnt(2)" : __VA_ARGS__); break;                 \
    case 3: asm volatile("s_waitcnt lgkmcnt(3)" : __VA_ARGS__); break;                 \
    case 4: asm volatile("s_waitcnt lgkmcnt(4)" : __VA_ARGS__); break;                 \
    case 5: asm volatile("s_waitcnt lgkmcnt(5)" : __VA_ARGS__); break;                 \
    case 6: asm volatile("s_waitcnt lgkmcnt(6)" : __VA_ARGS__); break;                 \
    case 7: asm volatile("s_waitcnt lgkmcnt(7)" : __VA_ARGS__); break;                 \
    case 8: asm volatile("s_waitcnt lgkmcnt(8)" : __VA_ARGS__); break;                 \
    case 9: asm volatile("s_waitcnt lgkmcnt(9)" : __VA_ARGS__); break;                 \
    case 10: asm volatile("s_waitcnt lgkmcnt(10)" : __VA_ARGS__); break;               \
    case 11: asm volatile("s_waitcnt lgkmcnt(11)" : __VA_ARGS__); break;               \
    case 12: asm volatile("s_waitcnt lgkmcnt(12)" : __VA_ARGS__); break;               \
    case 13: asm volatile("s_waitcnt lgkmcnt(13)" : __VA_ARGS__); break;               \
    case 14: asm volatile("s_waitcnt lgkmcnt(14)" : __VA_ARGS__); break;               \
    default: asm volatile("s_waitcnt lgkmcnt(15)" : __VA_ARGS__); break;               \
  }

template <typename T>
__device__ __forceinline__ void lds_wait(int n, T& x) {
  MSA_LGKM_SWITCH(n, "+v"(x))
}
template <typename T, typename U>
__device__ __forceinline__ void lds_wait(int n, T& x, U& y) {
  MSA_LGKM_SWITCH(n, "+v"(x), "+v"(y))
}
#undef MSA_LGKM_SWITCH

// Index of this lane's wavefront within the workgroup, as a value the
// compiler knows to be uniform: what is derived from it (row ranges, LDS
// destinations of direct-to-LDS loads, tile-visibility tests) then lives in
// scalar registers and costs no vector instructions per tile.
__device__ __forceinline__ int wave_index(int tid) {
  return __builtin_amdgcn_readfirstlane(tid >> 6);
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// MI355X dispatches workgroup i to XCD (i mod 8).  Renumber so that the
// workgroups an XCD runs are consecutive in the logical order, which keeps
// the data they share inside that XCD's L2.  Bijective for any count.
__device__ __forceinline__ int xcd_remap(int i, int count) {
  constexpr int kXcd = 8;
  const int xcd = i % kXcd;
  const int slot = i / kXcd;
  const int per = count / kXcd;
  const int rem = count % kXcd;
  return xcd * per + (xcd < rem ? xcd : rem) + slot;
}

}  // namespace msa
