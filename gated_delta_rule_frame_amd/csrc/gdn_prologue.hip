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
// group in flight.  Layout: per (batch, head) the pairs (fk, fq) of tokens
// -1 .. T (T + 2 pairs, the two pads zero), so that two neighbouring tokens'
// factors are one 16-byte load for any token pair a kernel stages.
#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr float kEps = 1e-6f;
constexpr int kTokensPerBlock = 16;   // 16 lane groups: 4 heads x 4 tokens, 4 rows each
constexpr int kHeadsPerBlock = 4;

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

// Block: 256 threads, lane group grp = threadIdx.x / 16 on head
// blockIdx.y * 4 + grp % 4 and tokens blockIdx.x * 16 + 4 (grp / 4) + j, j < 4,
// of batch blockIdx.z: the four groups of a wavefront read the same token of
// four neighbouring heads, one contiguous stretch of the [B, T, H, d] tensor
// (a token's row of q or k is U 16-byte pieces), and each group writes the
// factor pairs of four consecutive tokens (32 contiguous bytes).
template <bool BF16IN, int DK>
__global__ __launch_bounds__(256) void prologue_kernel(const uint4* __restrict__ q, const uint4* __restrict__ k,
                                                       float2* __restrict__ fac, long long T, int H) {
  constexpr int U = DK * (BF16IN ? 2 : 4) / 16;   // <= 32
  constexpr int NU = (U + 15) / 16;
  const int l = threadIdx.x & 15, grp = threadIdx.x >> 4;
  const int h = blockIdx.y * kHeadsPerBlock + (grp & 3), b = blockIdx.z;
  const long long t0 = (long long)blockIdx.x * kTokensPerBlock + 4 * (grp >> 2);
  float2* const fh = fac + ((long long)b * H + h) * (T + 2) + 1;   // pair of token 0
  float sk[4], sq[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const long long t = t0 + j, row = ((long long)b * T + t) * H + h;
    sk[j] = sq[j] = 0.f;
    if (t < T && h < H) {
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
    const float a = group16_sum(sk[j]), c = group16_sum(sq[j]);
    const long long t = t0 + j;
    if (l == 0 && t < T && h < H) {
      fh[t] = make_float2(1.f / __builtin_sqrtf(a / (float)DK + kEps), 1.f / __builtin_sqrtf(c + kEps));
      if (t == 0) fh[-1] = make_float2(0.f, 0.f);
      if (t == T - 1) fh[T] = make_float2(0.f, 0.f);
    }
  }
}

}  // namespace

size_t prologue_bytes(const Problem& p) {
  return p.prologue ? 2 * (size_t)p.B * p.H * (p.T + 2) * sizeof(float) : 0;
}

hipError_t prologue_launch(const Problem& p, const Tensors& t, float* fac, hipStream_t stream) {
  const dim3 grid((unsigned)((p.T + kTokensPerBlock - 1) / kTokensPerBlock),
                  (unsigned)((p.H + kHeadsPerBlock - 1) / kHeadsPerBlock), (unsigned)p.B);
  float2* f2 = reinterpret_cast<float2*>(fac);
  const uint4* q = static_cast<const uint4*>(t.q);
  const uint4* k = static_cast<const uint4*>(t.k);
  prof_begin(stream, GDN_KERNEL_PROLOGUE);
#define GDN_PRO_CASE(D)                                                                                   \
  case D:                                                                                                 \
    if (p.qkv_bf16)                                                                                       \
      hipLaunchKernelGGL((prologue_kernel<true, D>), grid, dim3(256), 0, stream, q, k, f2, p.T, \
                         p.H);                                                                   \
    else                                                                                                  \
      hipLaunchKernelGGL((prologue_kernel<false, D>), grid, dim3(256), 0, stream, q, k, f2, p.T, \
                         p.H);                                                                   \
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
