// MFMA tile helpers for gfx950 (CDNA4), wave64.
//
// The chunk kernels multiply fp16 operands with fp32 accumulation
// (v_mfma_f32_16x16x32_f16 runs at the bf16 rate on gfx950 and keeps three
// more mantissa bits for the intermediate operands); the split-precision
// segment chain uses the bf16 forms.
//
// Operand convention: one 16x16 output tile is D[m][n] = sum_k A[m][k] B[n][k];
// lane l supplies row (l % 16) of A and of B, with k in [8 (l/16), +8) for the
// 16x16x32 forms and k in [4 (l/16), +4) for the 16x16x16 forms (any k order
// shared by both operands gives the same sum).  Accumulator layout (both):
// lane l holds column n = l % 16 and rows m = 4 (l/16) + r, r = 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t hb;  // raw fp16 bits (chunk-kernel operands)
typedef uint16_t bh;  // raw bf16 bits

__device__ __forceinline__ hb f2h(float x) {
  const _Float16 h = static_cast<_Float16>(x);  // round to nearest even
  return __builtin_bit_cast(hb, h);
}

__device__ __forceinline__ bh f2bh(float x) {
  const __bf16 b = static_cast<__bf16>(x);      // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(bh, b);
}

__device__ __forceinline__ float bh2f(bh b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// Eight bf16 values (one 16-byte chunk) to eight fp16 values.  Exact for
// magnitudes in fp16's normal range; smaller ones become fp16 subnormals
// (absolute error below 6e-8).
__device__ __forceinline__ uint4 bf16x8_to_f16x8(uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(w[i] << 16), hi = __uint_as_float(w[i] & 0xffff0000u);
    o[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Eight bf16 values times s, rounded to the nearest fp16; with RELU, products
// below zero become zero (NaN stays NaN).
template <bool RELU>
__device__ __forceinline__ uint4 bf16x8_scaled_f16x8(uint4 v, float s) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float lo = __uint_as_float(w[i] << 16) * s, hi = __uint_as_float(w[i] & 0xffff0000u) * s;
    if constexpr (RELU) {
      lo = lo < 0.f ? 0.f : lo;
      hi = hi < 0.f ? 0.f : hi;
    }
    o[i] = static_cast<uint32_t>(f2h(lo)) | (static_cast<uint32_t>(f2h(hi)) << 16);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Ordering of LDS traffic between lanes of one wavefront.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace gdn
