// Feature prologue: per-token factors of the key features and the normalised
// queries.
//
// The key features are ReLU(RMSNorm(k)) over the d_k components of each
// (token, head) key with no learned weight, and the queries are L2-normalised
// ("SANA-WM: Efficient Minute-Scale World Modeling with Hybrid Linear
// Diffusion Transformer", summary page, section 3.2, "Algebraic Stabilization
// for Spatial Token Explosion" and the token-wise update).  Both are a
// positive per-row factor times the row (ReLU commutes with a positive
// factor), so this kernel only computes the factors
//     fk = 1 / sqrt(mean(k^2) + eps),   fq = 1 / sqrt(sum(q^2) + eps)
// into the workspace; the kernels that load q and k multiply by them (and
// apply the ReLU to keys) while staging, and the normalised tensors never
// reach memory.  One pass reads q and k once: 16 lanes per row, each lane
// one or two 16-byte pieces, a 16-lane shuffle reduction, four rows per lane
// group in flight.
#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr float kEps = 1e-6f;
constexpr int kRowsPerBlock = 64;   // 16 lane groups x 4 rows

__device__ __forceinline__ float sq_sum(uint4 u, bool bf16) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (bf16) {
      const float lo = __uint_as_float(w[i] << 16), hi = __uint_as_float(w[i] & 0xffff0000u);
      s = fmaf(lo, lo, s);
      s = fmaf(hi, hi, s);
    } else {
      const float x = __uint_as_float(w[i]);
      s = fmaf(x, x, s);
    }
  }
  return s;
}

__device__ __forceinline__ float group16_sum(float x) {
  x += __shfl_xor(x, 8, 16);
  x += __shfl_xor(x, 4, 16);
  x += __shfl_xor(x, 2, 16);
  x += __shfl_xor(x, 1, 16);
  return x;
}

// Block: 256 threads, rows blockIdx.x * 64 + 16 j + (threadIdx.x / 16), j < 4
// (each wavefront reads 4 consecutive rows per j).  U 16-byte pieces per row.
template <bool BF16IN, int DK>
__global__ __launch_bounds__(256) void prologue_kernel(const uint4* __restrict__ q, const uint4* __restrict__ k,
                                                       float* __restrict__ fk, float* __restrict__ fq,
                                                       long long rows) {
  constexpr int U = DK * (BF16IN ? 2 : 4) / 16;   // <= 32
  constexpr int NU = (U + 15) / 16;
  const int l = threadIdx.x & 15;
  const long long r0 = (long long)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 4);
  float sk[4], sq[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const long long row = r0 + 16 * j;
    sk[j] = sq[j] = 0.f;
    if (row < rows) {
#pragma unroll
      for (int i = 0; i < NU; ++i) {
        const int u = l + 16 * i;
        if (u < U) {
          sk[j] += sq_sum(k[row * U + u], BF16IN);
          sq[j] += sq_sum(q[row * U + u], BF16IN);
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a = group16_sum(sk[j]), b = group16_sum(sq[j]);
    const long long row = r0 + 16 * j;
    if (l == 0 && row < rows) {
      fk[row] = 1.f / __builtin_sqrtf(a / (float)DK + kEps);
      fq[row] = 1.f / __builtin_sqrtf(b + kEps);
    }
  }
}

}  // namespace

size_t prologue_bytes(const Problem& p) {
  return p.prologue ? 2 * (size_t)p.B * p.T * p.H * sizeof(float) : 0;
}

hipError_t prologue_launch(const Problem& p, const Tensors& t, float* fac, hipStream_t stream) {
  const long long rows = (long long)p.B * p.T * p.H;
  const long long blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  float* fk = fac;
  float* fq = fac + rows;
  const uint4* q = static_cast<const uint4*>(t.q);
  const uint4* k = static_cast<const uint4*>(t.k);
  prof_begin(stream, GDN_KERNEL_PROLOGUE);
#define GDN_PRO_CASE(D)                                                                                   \
  case D:                                                                                                 \
    if (p.qkv_bf16)                                                                                       \
      hipLaunchKernelGGL((prologue_kernel<true, D>), dim3((unsigned)blocks), dim3(256), 0, stream, q, k, \
                         fk, fq, rows);                                                                   \
    else                                                                                                  \
      hipLaunchKernelGGL((prologue_kernel<false, D>), dim3((unsigned)blocks), dim3(256), 0, stream, q, k, \
                         fk, fq, rows);                                                                   \
    break;
  switch (p.dk) {
    GDN_PRO_CASE(16) GDN_PRO_CASE(32) GDN_PRO_CASE(48) GDN_PRO_CASE(64)
    GDN_PRO_CASE(80) GDN_PRO_CASE(96) GDN_PRO_CASE(112) GDN_PRO_CASE(128)
    default: return hipErrorInvalidValue;
  }
#undef GDN_PRO_CASE
  const hipError_t e = hipGetLastError();
  prof_end(stream, GDN_KERNEL_PROLOGUE);
  return e;
}

}  // namespace gdn
