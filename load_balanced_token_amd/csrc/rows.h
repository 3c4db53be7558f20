// Row-movement helpers shared by the dispatch/combine and training kernels:
// native vector types, scalar-base addressing, XCD-aware workgroup order and
// bf16 <-> fp32 conversion.
#pragma once
#include "lbt_internal.h"

namespace lbt {

// Native clang vector types: the nontemporal builtins take these, not
// HIP_vector_type.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));


// Element `byte_off` bytes into a row that starts at a wave-uniform address:
// a uniform 64-bit base plus an unsigned 32-bit lane offset lets the
// compiler use scalar-base addressing instead of a 64-bit VGPR address per
// access.
template <typename T>
__device__ __forceinline__ const T* at_bytes(const void* base, uint32_t byte_off) {
  return reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + byte_off);
}
template <typename T>
__device__ __forceinline__ T* at_bytes(void* base, uint32_t byte_off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(base) + byte_off);
}

// Workgroup i runs on XCD i % 8; give each XCD a contiguous range of tokens
// so that one XCD's L2 sees neighbouring rows.  A bijection on [0, G).
__device__ __forceinline__ int xcd_contiguous(int i, int G) {
  const int q = G / 8, rem = G % 8, x = i % 8, pos = i / 8;
  return x * q + min(x, rem) + pos;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if (f != f) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

}  // namespace lbt
