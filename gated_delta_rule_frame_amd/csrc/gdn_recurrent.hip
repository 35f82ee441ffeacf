// Token-sequential gated delta rule on gfx950: the reference GPU path.
//
// It runs the token-wise Gated DeltaNet update ("SANA-WM: Efficient
// Minute-Scale World Modeling with Hybrid Linear Diffusion Transformer",
// summary page, section 3.2, token-wise update) literally, token after token,
// in fp32 on the vector ALUs.  It serves fp32 inputs (whose tolerance needs
// fp32 products) and is the permanent GPU cross-check of the chunked path.
//
// Work split: one wavefront per (batch, head, 16 value columns).  The state
// slice H[:, cols] (d_k x 16, fp32) stays in VGPRs for the whole sequence:
// lane l owns column (l % 16) and rows r = (l / 16) + 4 m.  The two dot
// products of a token (k^T H and q^T H) are a per-lane partial sum followed by
// a 4-way cross-lane reduction (lanes l, l^16, l^32, l^48).  Tokens are staged
// through LDS in blocks of 32.  With the feature prologue, keys and queries
// are multiplied by their per-(token, head) factors on load and the keys pass
// through ReLU.
#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kCols = 16;  // value columns per wavefront
constexpr int kTok = 32;   // tokens staged per LDS block

// out_mode: 0 write `out`; 1 write the fp32 partial to `acc`; 2 add `acc`,
// then write `out`.
template <bool BF16IN, int DK>
__global__ __launch_bounds__(64) void recurrent_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const float* h0,
    void* __restrict__ out, float* hT, float* __restrict__ acc, long long T, int H, int DV,
    int reverse, int out_mode, int out_bf16, float key_scale, long long reset_first, long long reset_every,
    const float* __restrict__ fac) {
  constexpr int R = DK / 4;
  const int lane = threadIdx.x;
  const int c = lane & 15, r0 = lane >> 4;
  const int col0 = blockIdx.x * kCols;
  const int h = blockIdx.y, b = blockIdx.z;

  __shared__ float ks[kTok][DK];
  __shared__ float qs[kTok][DK];
  __shared__ float vs[kTok][kCols];
  __shared__ float gs[kTok], bs[kTok];

  const size_t sbase = ((size_t)b * H + h) * DK * DV;
  float st[R];
#pragma unroll
  for (int m = 0; m < R; ++m)
    st[m] = h0 ? h0[sbase + (size_t)(r0 + 4 * m) * DV + col0 + c] : 0.f;

  for (long long t0 = 0; t0 < T; t0 += kTok) {
    const int nt = (int)((T - t0) < kTok ? (T - t0) : kTok);
    __syncthreads();
    for (int idx = lane; idx < nt * DK; idx += 64) {
      const int j = idx / DK, i = idx % DK;
      const long long tau = reverse ? T - 1 - (t0 + j) : t0 + j;
      const size_t row = ((size_t)b * T + tau) * H + h, off = row * DK + i;
      float kv = load_scalar<BF16IN>(k, off), qv = load_scalar<BF16IN>(q, off);
      if (fac) {
        // (fk, fq) of token tau: pair tau + 1 of this (batch, head)
        const float* f = fac + 2 * (((size_t)b * H + h) * (T + 2) + tau + 1);
        kv *= f[0];
        kv = kv < 0.f ? 0.f : kv;
        qv *= f[1];
      }
      ks[j][i] = kv * key_scale;
      qs[j][i] = qv;
    }
    for (int idx = lane; idx < nt * kCols; idx += 64) {
      const int j = idx / kCols, cc = idx % kCols;
      const long long tau = reverse ? T - 1 - (t0 + j) : t0 + j;
      vs[j][cc] = load_scalar<BF16IN>(v, (((size_t)b * T + tau) * H + h) * DV + col0 + cc);
    }
    if (lane < nt) {
      const long long tau = reverse ? T - 1 - (t0 + lane) : t0 + lane;
      const size_t go = ((size_t)b * T + tau) * H + h;
      gs[lane] = g[go];
      bs[lane] = beta[go];
    }
    __syncthreads();
    for (int j = 0; j < nt; ++j) {
      if (reset_every > 0) {
        // chunk-causal reversed scan: it restarts from zero at the last
        // token of every chunk (chunk ends at reset_first + m reset_every)
        const long long e1 = T - (t0 + j);   // one past the token, in original order
        if (e1 == reset_first || (e1 > reset_first && (e1 - reset_first) % reset_every == 0)) {
#pragma unroll
          for (int m = 0; m < R; ++m) st[m] = 0.f;
        }
      }
      const float a = expf(gs[j]);
      float p = 0.f;
#pragma unroll
      for (int m = 0; m < R; ++m) {
        st[m] *= a;
        p = fmaf(ks[j][r0 + 4 * m], st[m], p);
      }
      p += __shfl_xor(p, 16);
      p += __shfl_xor(p, 32);
      const float e = (vs[j][c] - p) * bs[j];
      float o = 0.f;
#pragma unroll
      for (int m = 0; m < R; ++m) {
        st[m] = fmaf(ks[j][r0 + 4 * m], e, st[m]);
        o = fmaf(qs[j][r0 + 4 * m], st[m], o);
      }
      o += __shfl_xor(o, 16);
      o += __shfl_xor(o, 32);
      if (r0 == 0) {
        const long long tau = reverse ? T - 1 - (t0 + j) : t0 + j;
        const size_t oo = (((size_t)b * T + tau) * H + h) * DV + col0 + c;
        if (out_mode == 1) {
          acc[oo] = o;
        } else {
          if (out_mode == 2) o += acc[oo];
          store_scalar(out, oo, o, out_bf16 != 0);
        }
      }
    }
  }
  if (hT) {
#pragma unroll
    for (int m = 0; m < R; ++m) hT[sbase + (size_t)(r0 + 4 * m) * DV + col0 + c] = st[m];
  }
}

template <bool BF16IN>
hipError_t launch_dk(const Problem& p, const Tensors& t, bool reverse, const float* h0, int out_mode,
                     float* acc, const float* fac, bool write_state, hipStream_t stream, long long reset_first = 0,
                     long long reset_every = 0) {
  dim3 grid(p.dv / kCols, p.H, p.B), block(64);
  float* hT = write_state ? t.hT : nullptr;
  prof_begin(stream, GDN_KERNEL_RECURRENT);
#define GDN_REC_CASE(D)                                                                       \
  case D:                                                                                     \
    hipLaunchKernelGGL((recurrent_kernel<BF16IN, D>), grid, block, 0, stream, t.q, t.k, t.v, \
                       t.g, t.beta, h0, t.out,           hT, acc, p.T, p.H, p.dv,  \
                       reverse ? 1 : 0, out_mode, p.out_bf16 ? 1 : 0, p.key_scale,            \
                       reset_first, reset_every, fac);                                        \
    break;
  switch (p.dk) {
    GDN_REC_CASE(16) GDN_REC_CASE(32) GDN_REC_CASE(48) GDN_REC_CASE(64)
    GDN_REC_CASE(80) GDN_REC_CASE(96) GDN_REC_CASE(112) GDN_REC_CASE(128)
    default: return hipErrorInvalidValue;
  }
#undef GDN_REC_CASE
  const hipError_t e = hipGetLastError();
  prof_end(stream, GDN_KERNEL_RECURRENT);
  return e;
}

}  // namespace

namespace {
// The bidirectional sum goes through an fp32 accumulator so that the output
// is rounded once; the prologue factors follow it.
size_t acc_bytes(const Problem& p, int direction) {
  if (direction != GDN_BIDIRECTIONAL && direction != GDN_CHUNK_CAUSAL) return 0;
  return align_up((size_t)p.B * p.T * p.H * p.dv * sizeof(float), 256);
}
}  // namespace

size_t recurrent_workspace(const Problem& p, int direction) {
  return acc_bytes(p, direction) + prologue_bytes(p);
}

hipError_t recurrent_launch(const Problem& p, int direction, const Tensors& t, void* workspace,
                            hipStream_t stream) {
  float* acc = static_cast<float*>(workspace);
  float* fac = p.prologue ? reinterpret_cast<float*>(static_cast<char*>(workspace) + acc_bytes(p, direction)) : nullptr;
  if (fac) {
    const hipError_t e = prologue_launch(p, t, fac, stream);
    if (e != hipSuccess) return e;
  }
  auto go = [&](bool reverse, const float* h0, int mode, bool state, long long rf = 0, long long re = 0) {
    return p.qkv_bf16 ? launch_dk<true>(p, t, reverse, h0, mode, acc, fac, state, stream, rf, re)
                      : launch_dk<false>(p, t, reverse, h0, mode, acc, fac, state, stream, rf, re);
  };
  if (direction == GDN_FORWARD) return go(false, t.h0, 0, true);
  // Backward-only mode: initial_state seeds the reversed scan.
  if (direction == GDN_BACKWARD) return go(true, t.h0, 0, true);
  // Bidirectional: forward scan from initial_state into the fp32 accumulator,
  // then the reversed scan from zero adds to it and writes `out`.
  hipError_t e = go(false, t.h0, 1, true);
  if (e != hipSuccess) return e;
  if (direction == GDN_CHUNK_CAUSAL)   // reversed scan confined to each chunk of frames
    return go(true, nullptr, 2, false, (long long)p.first_chunk_frames * p.S, (long long)p.chunk_frames * p.S);
  return go(true, nullptr, 2, false);
}

}  // namespace gdn
