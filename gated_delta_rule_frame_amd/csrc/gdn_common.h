// Small device helpers shared by the libgdn kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// bf16 <-> fp32.  bf16 is the upper half of an IEEE fp32 word, so widening is
// exact; narrowing rounds to nearest, ties to even, and keeps NaN quiet.
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7f800000u) == 0x7f800000u)                      // Inf or NaN
    return static_cast<uint16_t>((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <bool BF16>
__device__ __forceinline__ float load_scalar(const void* p, size_t i) {
  if constexpr (BF16) return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
  else return static_cast<const float*>(p)[i];
}

__device__ __forceinline__ void store_scalar(void* p, size_t i, float x, bool bf16) {
  if (bf16) static_cast<uint16_t*>(p)[i] = f32_to_bf16_bits(x);
  else static_cast<float*>(p)[i] = x;
}

}  // namespace gdn
