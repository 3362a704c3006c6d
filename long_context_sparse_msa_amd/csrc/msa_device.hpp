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
