// Frame-chunked gated delta rule forward on gfx950 with MFMA.
//
// The token-wise update ("SANA-WM: Efficient Minute-Scale World Modeling with
// Hybrid Linear Diffusion Transformer", summary page, section 3.2, token-wise
// Gated DeltaNet update) composes, over a run of tokens, into a product of
// rank-1 corrections of the identity.  This file evaluates that product in
// blocks instead of token by token.  The algebra (exact up to rounding):
//
// Sub-chunk of n <= 64 tokens in scan order, gates g_i, inclusive cumsum G_i,
// E_ij = exp(G_i - G_j) (only i >= j is ever evaluated, so every exponent is
// <= 0 on the documented domain), keys scaled by c = key_scale:
//     A   = strict_lower(c^2 diag(beta) K K^T * E)                     (64x64)
//     Tm  = (I + A)^-1                       (blocked triangular inverse)
//     W   = c Tm diag(beta e^G) K,   U = Tm diag(beta) V              (WY/UT form)
//     V'  = U - W H                          (values minus the state's prediction)
//     O   = diag(e^G) Q H + (c tril(Q K^T) * E) V'       (read after write)
//     H  <- e^{G_n} H + c K^T diag(e^{G_n - G}) V'
//
// Schedule.  The token axis is cut, in original order, into segments of L
// tokens (a multiple of 64) and each segment into 64-token sub-chunks; a scan
// direction visits both in its own order.  Three launches per call:
//   1. seg_map_kernel   (parallel over segments): the segment's affine state
//      map H_end = P H_start + Q, by running the sub-chunk chain on the
//      augmented state X = [P | Q] from [I | 0] with values [0 | V];
//   2. seg_chain_kernel (serial over segments, parallel over heads and value
//      columns): H_{s+1} = P_s H_s + Q_s in split-bf16 (hi + lo) MFMA, i.e. the
//      prefix composition of the segments' transition maps;
//   3. seg_out_kernel   (parallel over segments): each segment re-run from its
//      true start state, writing outputs (both scan directions of a segment in
//      one workgroup, summed before the single store) and the final state.
// All states and accumulations are fp32.  MFMA operands of the chunk kernels
// are fp16: the bf16 inputs convert to fp16 exactly (in fp16's normal range)
// and each rounded intermediate (Tm, W, H, V', P) keeps 11 significant bits
// instead of bf16's 8, which holds the result well inside the bf16-input
// tolerance at no extra MFMA work.  Precondition of this path: inputs and
// intermediate magnitudes stay below fp16's maximum (65504).
#include "gdn_common.h"
#include "gdn_internal.h"
#include "gdn_mfma.h"

#include <atomic>

namespace gdn {
namespace {

constexpr int CH = 64;          // sub-chunk tokens
constexpr int NT = 256;         // threads per workgroup of the map and output kernels
constexpr int NW = NT / 64;     // wavefronts per workgroup
constexpr int NTC = 256;        // threads per workgroup of the chain kernel
constexpr int NWC = NTC / 64;
constexpr int LDT = CH + 8;     // row stride (elements) of token-contracted fp16 matrices
constexpr int LDA = CH + 4;     // row stride of the fp32 A matrix
constexpr float kLog2e = 1.4426950408889634f;

std::atomic<int> g_segment_override{0};


struct Args {
  const bh* q;
  const bh* k;
  const bh* v;
  const float* g;
  const float* beta;
  const float* h0;      // initial state or null
  void* out;
  float* acc;           // fp32 partial of the reversed scan (BIDIR)
  float* hT;            // final state or null
  float* maps;          // [ndir][B][H][NS-1][DK][DK+DV]
  float* starts;        // [ndir][B][H][NS][DK][DV]
  long long T;
  int B, H, L, NS;
  int dirs;             // bit 0: forward scan, bit 1: reversed scan
  int out_bf16;
  float c;              // key scale
};

// Wavefront index as a wave-uniform (scalar) value, so that branches on it are
// scalar branches rather than per-lane exec masking.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ int dir_of_slot(int dirs, int slot) {
  // slot 0 is the forward scan when present
  return (dirs & 1) ? (slot == 0 ? 0 : 1) : 1;
}
__device__ __forceinline__ int slot_of_dir(int dirs, int dir) { return (dir == 1 && (dirs & 1)) ? 1 : 0; }

// Shared-memory layout of a workgroup.  OUT: the output pass (else the map
// pass).  Only operands shared by all wavefronts live here; each wavefront's
// state strips, U, V' and outputs stay in registers.
template <int D, bool OUT>
struct Lay {
  static constexpr int LDK = D + 8;    // row stride of d-contracted matrices
  static constexpr int KR = CH * LDK * 2;
  static constexpr int QR = OUT ? CH * LDK * 2 : 0;
  static constexpr int KT = D * LDT * 2;
  static constexpr int VT = D * LDT * 2;
  static constexpr int AF = CH * LDA * 4;
  static constexpr int SQ = CH * LDT * 2;
  static constexpr int NSQ = OUT ? 5 : 4;
  static constexpr int o_kr = 0;
  static constexpr int o_qr = o_kr + KR;
  static constexpr int o_kt = o_qr + QR;
  static constexpr int o_vt = o_kt + KT;
  static constexpr int o_af = o_vt + VT;
  static constexpr int o_sq = o_af + AF;
  static constexpr int o_g2 = o_sq + NSQ * SQ;
  static constexpr int o_bt = o_g2 + CH * 4;
  static constexpr int BYTES = o_bt + CH * 4;
  static_assert(BYTES <= 160 * 1024, "workgroup LDS budget exceeded");
  static_assert(KR % 16 == 0 && KT % 16 == 0 && AF % 16 == 0 && SQ % 16 == 0, "alignment");
};

template <int D, bool OUT>
struct Smem {
  using L = Lay<D, OUT>;
  hb *kr, *qr, *kt, *vt, *p, *ab, *tbt, *t1, *t2;
  float *af, *g2, *bt;
  __device__ explicit Smem(char* s) {
    kr = reinterpret_cast<hb*>(s + L::o_kr);
    qr = reinterpret_cast<hb*>(s + L::o_qr);
    kt = reinterpret_cast<hb*>(s + L::o_kt);
    vt = reinterpret_cast<hb*>(s + L::o_vt);
    af = reinterpret_cast<float*>(s + L::o_af);
    hb* sq = reinterpret_cast<hb*>(s + L::o_sq);
    ab = sq;
    tbt = sq + CH * LDT;
    t1 = sq + 2 * CH * LDT;
    t2 = sq + 3 * CH * LDT;
    p = OUT ? sq + 4 * CH * LDT : nullptr;
    g2 = reinterpret_cast<float*>(s + L::o_g2);
    bt = reinterpret_cast<float*>(s + L::o_bt);
  }
};

// Lower-triangular 16x16-tile pairs (a <= b) of a 4x4 tile grid.
__device__ __forceinline__ void tri_pair(int t, int& a, int& b) {
  constexpr int A[10] = {0, 0, 0, 0, 1, 1, 1, 2, 2, 3};
  constexpr int B[10] = {0, 1, 2, 3, 1, 2, 3, 2, 3, 3};
  a = A[t];
  b = B[t];
}

__device__ __forceinline__ void store4_h(hb* dst, float a, float b, float c, float d) {
  uint2 u;
  u.x = static_cast<uint32_t>(f2h(a)) | (static_cast<uint32_t>(f2h(b)) << 16);
  u.y = static_cast<uint32_t>(f2h(c)) | (static_cast<uint32_t>(f2h(d)) << 16);
  *reinterpret_cast<uint2*>(dst) = u;
}

// --- register-operand MFMA helpers -----------------------------------------
// A 16x16 accumulator tile X (lane l: X[4(l/16) + r][l % 16]) converted to
// fp16 is directly the B operand of a 16x16x16 product contracting over X's
// rows.  Two such tiles (rows 0-15 and 16-31 of the contraction) form the B
// operand of a 16x16x32 product whose k order is {4g..4g+3, 16+4g..16+4g+3}
// for lane group g; the A operand is then read from LDS in that same order.

__device__ __forceinline__ f16x4_t ld4(const hb* p) { return *reinterpret_cast<const f16x4_t*>(p); }
__device__ __forceinline__ f16x8_t ld8(const hb* p) { return *reinterpret_cast<const f16x8_t*>(p); }
__device__ __forceinline__ f16x8_t cat8(f16x4_t x, f16x4_t y) {
  return __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f16x4_t tof16(f32x4 v) {
  f16x4_t h;
  h[0] = static_cast<_Float16>(v[0]);
  h[1] = static_cast<_Float16>(v[1]);
  h[2] = static_cast<_Float16>(v[2]);
  h[3] = static_cast<_Float16>(v[3]);
  return h;
}
__device__ __forceinline__ f32x4 mfma32(f16x8_t x, f16x8_t y, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(x, y, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(f16x4_t x, f16x4_t y, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(x, y, c, 0, 0, 0);
}

// acc + x * y for a K = 16 step.  With this toolchain a dependent accumulator
// chain that mixes the 16x16x32 and 16x16x16 MFMA shapes produces wrong sums
// (measured on gfx950: large errors on a fraction of the elements), while each
// shape alone and independent accumulators are exact.  So a K = 16 step always
// starts a fresh accumulator and is added on the VALU; every accumulator chain
// uses one MFMA shape only.
__device__ __forceinline__ f32x4 mfma16_add(f16x4_t x, f16x4_t y, f32x4 acc) {
  return acc + mfma16(x, y, zero4());
}

// A fragment of k tiles (q, q + 1) in the register-B order, or of tile q alone.
__device__ __forceinline__ f16x8_t fragA2(const hb* arow, int q, int g) {
  return cat8(ld4(arow + 16 * q + 4 * g), ld4(arow + 16 * q + 16 + 4 * g));
}
__device__ __forceinline__ f16x4_t fragA1(const hb* arow, int q, int g) { return ld4(arow + 16 * q + 4 * g); }

__device__ __forceinline__ f16x8_t tof16x8(f32x4 u, f32x4 v) { return cat8(tof16(u), tof16(v)); }
__device__ __forceinline__ f16x4_t lo4(f16x8_t v) { return __builtin_shufflevector(v, v, 0, 1, 2, 3); }

// acc[j] += A[row(lane), 0:16 n] * B_j for all SPW strips of the wavefront,
// contracting over NP pairs of fp16 accumulator tiles bp[j][p] = (tile 2p,
// tile 2p + 1) and, if TAIL, one more tile bt[j].  Each A fragment is read from
// LDS once and used for every strip.  Strips past the state's width are
// computed on clamped data and never stored: a wave with fewer real strips
// would wait at the next barrier anyway, and branch-free code keeps the
// accumulators in place (no merge copies).
template <int SPW, int NP, bool TAIL>
__device__ __forceinline__ void mma_dB(const hb* arow, const f16x8_t (*bp)[NP > 0 ? NP : 1], const f16x4_t* bt,
                                       int g, f32x4* acc) {
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const f16x8_t x = fragA2(arow, 2 * p, g);
#pragma unroll
    for (int j = 0; j < SPW; ++j) acc[j] = mfma32(x, bp[j][p], acc[j]);
  }
  if constexpr (TAIL) {
    const f16x4_t x = fragA1(arow, 2 * NP, g);
#pragma unroll
    for (int j = 0; j < SPW; ++j) acc[j] = mfma16_add(x, bt[j], acc[j]);
  }
}

// Same, contracting over the first n (1..4) token tiles held as the pairs
// vp[j][0] = (tiles 0, 1) and vp[j][1] = (tiles 2, 3).
template <int SPW>
__device__ __forceinline__ void mma_tB(const hb* arow, const f16x8_t (*vp)[2], int n, int g, f32x4* acc) {
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    if (2 * p + 1 < n) {
      const f16x8_t x = fragA2(arow, 2 * p, g);
#pragma unroll
      for (int j = 0; j < SPW; ++j) acc[j] = mfma32(x, vp[j][p], acc[j]);
    } else if (2 * p < n) {
      const f16x4_t x = fragA1(arow, 2 * p, g);
#pragma unroll
      for (int j = 0; j < SPW; ++j) acc[j] = mfma16_add(x, lo4(vp[j][p]), acc[j]);
    }
  }
}

// acc += A[row(lane), 0:16 n] * B[col(lane), 0:16 n]^T with both rows in LDS.
__device__ __forceinline__ f32x4 mma_lds(const hb* arow, const hb* brow, int n, int g, f32x4 acc) {
#pragma unroll
  for (int q = 0; q < 8; q += 2) {
    if (q + 1 < n)
      acc = mfma32(ld8(arow + 16 * q + 8 * g), ld8(brow + 16 * q + 8 * g), acc);
    else if (q < n)
      acc = mfma16_add(ld4(arow + 16 * q + 4 * g), ld4(brow + 16 * q + 4 * g), acc);
  }
  return acc;
}

// Global token index of scan-local row i of a sub-chunk [t0, t0 + n).
__device__ __forceinline__ long long token_of(long long t0, int n, bool rev, int i) {
  return rev ? t0 + n - 1 - i : t0 + i;
}

// --- per-sub-chunk preparation (shared by all wavefronts) -------------------

// Per-thread staging registers of one sub-chunk: a 4-token x 8-component
// block of K, V (and Q) and one token's log-gate and beta.  Loading into
// registers is split from writing LDS so that the next sub-chunk's global
// loads are in flight while the current one is being computed.
struct Stage {
  uint4 k[4], v[4], q[4];
  float g, b;
};

// Issue the global loads of sub-chunk [t0, t0 + n) (rows in scan order,
// zero-padded to 64 tokens).
template <int D, bool OUT>
__device__ __forceinline__ void fetch_subchunk(const Args& a, int b, int h, long long t0, int n, bool rev,
                                               Stage& st) {
  constexpr int C8 = D / 8;
  const int tid = threadIdx.x;
  if (tid < 16 * C8) {
    const int i4 = tid / C8, c8 = tid % C8;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * i4 + r;
      st.k[r] = st.v[r] = st.q[r] = make_uint4(0u, 0u, 0u, 0u);
      if (i < n) {
        const size_t off = ((size_t)((size_t)b * a.T + token_of(t0, n, rev, i)) * a.H + h) * D + 8 * c8;
        st.k[r] = *reinterpret_cast<const uint4*>(a.k + off);
        st.v[r] = *reinterpret_cast<const uint4*>(a.v + off);
        if constexpr (OUT) st.q[r] = *reinterpret_cast<const uint4*>(a.q + off);
      }
    }
  }
  st.g = 0.f;
  st.b = 0.f;
  if (tid < 64 && tid < n) {
    const size_t go = ((size_t)b * a.T + token_of(t0, n, rev, tid)) * a.H + h;
    st.g = a.g[go];
    st.b = a.beta[go];
  }
}

__device__ __forceinline__ uint2 pack4(hb x, hb y, hb z, hb w) {
  return make_uint2(static_cast<uint32_t>(x) | (static_cast<uint32_t>(y) << 16),
                    static_cast<uint32_t>(z) | (static_cast<uint32_t>(w) << 16));
}

// Write the staged sub-chunk into LDS as fp16 (K and Q row-major, K and V
// transposed) and form the scan-order gate cumsum (log2 units) and beta.
template <int D, bool OUT>
__device__ __forceinline__ void stage_subchunk(const Smem<D, OUT>& S, const Stage& st) {
  using L = Lay<D, OUT>;
  constexpr int C8 = D / 8;
  const int tid = threadIdx.x;
  if (tid < 16 * C8) {
    const int i4 = tid / C8, c8 = tid % C8;
    uint4 kh[4], vh[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      kh[r] = bf16x8_to_f16x8(st.k[r]);
      vh[r] = bf16x8_to_f16x8(st.v[r]);
      *reinterpret_cast<uint4*>(S.kr + (4 * i4 + r) * L::LDK + 8 * c8) = kh[r];
      if constexpr (OUT) *reinterpret_cast<uint4*>(S.qr + (4 * i4 + r) * L::LDK + 8 * c8) = bf16x8_to_f16x8(st.q[r]);
    }
    const hb* ke[4] = {reinterpret_cast<const hb*>(&kh[0]), reinterpret_cast<const hb*>(&kh[1]),
                       reinterpret_cast<const hb*>(&kh[2]), reinterpret_cast<const hb*>(&kh[3])};
    const hb* ve[4] = {reinterpret_cast<const hb*>(&vh[0]), reinterpret_cast<const hb*>(&vh[1]),
                       reinterpret_cast<const hb*>(&vh[2]), reinterpret_cast<const hb*>(&vh[3])};
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      *reinterpret_cast<uint2*>(S.kt + (8 * c8 + u) * LDT + 4 * i4) = pack4(ke[0][u], ke[1][u], ke[2][u], ke[3][u]);
      *reinterpret_cast<uint2*>(S.vt + (8 * c8 + u) * LDT + 4 * i4) = pack4(ve[0][u], ve[1][u], ve[2][u], ve[3][u]);
    }
  }
  if (tid < 64) {
    float s = st.g * kLog2e;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const float t = __shfl_up(s, d);
      if (tid >= d) s += t;
    }
    S.g2[tid] = s;
    S.bt[tid] = st.b;
  }
}

// Gram products of the staged sub-chunk: the strictly lower gated A (fp32 and
// fp16) and, for the output pass, the gated causal P = c tril(Q K^T) * E.
template <int D, bool OUT>
__device__ void gram_stage(const Args& a, const Smem<D, OUT>& S) {
  using L = Lay<D, OUT>;
  const int wave = wave_id(), lane = threadIdx.x & 63, g = lane >> 4;
  const float c2 = a.c * a.c;
  for (int t = wave; t < 10; t += NW) {
    int ta, tb;
    tri_pair(t, ta, tb);
    const int x = tb * 16 + (lane & 15);           // A/P row (scan-local token)
    const int y0 = ta * 16 + 4 * g;                // first of the lane's 4 columns
    const float gx = S.g2[x], bx = S.bt[x];
    // lane holds K_{y0+r} . K_x (symmetric Gram) and K_{y0+r} . Q_x
    const hb* ka = S.kr + (ta * 16 + (lane & 15)) * L::LDK;
    const f32x4 s = mma_lds(ka, S.kr + x * L::LDK, D / 16, g, zero4());
    float av[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int y = y0 + r;
      av[r] = (x > y) ? c2 * bx * s[r] * exp2f(gx - S.g2[y]) : 0.f;
    }
    *reinterpret_cast<float4*>(S.af + x * LDA + y0) = make_float4(av[0], av[1], av[2], av[3]);
    store4_h(S.ab + x * LDT + y0, av[0], av[1], av[2], av[3]);
    if constexpr (OUT) {
      const f32x4 z = mma_lds(ka, S.qr + x * L::LDK, D / 16, g, zero4());
      float pv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int y = y0 + r;
        pv[r] = (x >= y) ? a.c * z[r] * exp2f(gx - S.g2[y]) : 0.f;
      }
      store4_h(S.p + x * LDT + y0, pv[0], pv[1], pv[2], pv[3]);
    }
  }
}

// Diagonal 16x16 blocks of Tm = (I + A)^-1 by forward substitution in fp32
// (one wavefront: lane = (block, column)).  Writes Tm_ii row-major into the
// diagonal blocks of ab, column-major into tbt, and the scaled copies
// t1 = Tm diag(beta), t2 = c Tm diag(beta e^G).
template <int D, bool OUT>
__device__ void diag_inverse(const Args& a, const Smem<D, OUT>& S) {
  const int lane = threadIdx.x & 63;
  const int blk = lane >> 4, cc = lane & 15;
  const float* A0 = S.af + (16 * blk) * LDA + 16 * blk;
  float t[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float s = (r == cc) ? 1.f : 0.f;
#pragma unroll
    for (int k = 0; k < r; ++k) s = fmaf(-A0[r * LDA + k], t[k], s);
    t[r] = s;
  }
  const int col = 16 * blk + cc;
  const float bc = S.bt[col], ec = a.c * bc * exp2f(S.g2[col]);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = 16 * blk + r;
    S.ab[row * LDT + col] = f2h(t[r]);
    S.t1[row * LDT + col] = f2h(t[r] * bc);
    S.t2[row * LDT + col] = f2h(t[r] * ec);
  }
#pragma unroll
  for (int r = 0; r < 16; r += 4) store4_h(S.tbt + col * LDT + 16 * blk + r, t[r], t[r + 1], t[r + 2], t[r + 3]);
}

// Off-diagonal blocks of Tm, one block column per wavefront (waves 0..2):
// Tm_{ib,jb} = -Tm_{ib,ib} sum_{kb=jb}^{ib-1} A_{ib,kb} Tm_{kb,jb}.
template <int D, bool OUT>
__device__ void offdiag_inverse(const Args& a, const Smem<D, OUT>& S) {
  const int wave = wave_id(), lane = threadIdx.x & 63, g = lane >> 4;
  if (wave >= 3) return;
  const int jb = wave;
  hb* rt = reinterpret_cast<hb*>(S.af) + wave * 16 * LDT;   // R^T scratch (A is dead now)
  const int col = 16 * jb + (lane & 15);
  const float bc = S.bt[col], ec = a.c * bc * exp2f(S.g2[col]);
  for (int ib = jb + 1; ib < 4; ++ib) {
    const hb* arow = S.ab + (16 * ib + (lane & 15)) * LDT + 16 * jb;
    const f32x4 R = mma_lds(arow, S.tbt + col * LDT + 16 * jb, ib - jb, g, zero4());
    store4_h(rt + (lane & 15) * LDT + 4 * g, R[0], R[1], R[2], R[3]);
    wave_lds_sync();
    const f32x4 Dv = mma_lds(S.ab + (16 * ib + (lane & 15)) * LDT + 16 * ib, rt + (lane & 15) * LDT, 1, g,
                             zero4());
    const int row0 = 16 * ib + 4 * g;
    store4_h(S.tbt + col * LDT + row0, -Dv[0], -Dv[1], -Dv[2], -Dv[3]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      S.t1[(row0 + r) * LDT + col] = f2h(-Dv[r] * bc);
      S.t2[(row0 + r) * LDT + col] = f2h(-Dv[r] * ec);
    }
    wave_lds_sync();
  }
}

// -W rows into kr:  W = t2 K, computed as W^T = K^T t2^T so that each lane
// stores four consecutive d entries of one token row.
template <int D, bool OUT>
__device__ void w_stage(const Smem<D, OUT>& S) {
  using L = Lay<D, OUT>;
  const int wave = wave_id(), lane = threadIdx.x & 63, g = lane >> 4;
  for (int t = wave; t < (D / 16) * 4; t += NW) {
    const int md = t >> 2, nt = t & 3;
    const f32x4 w = mma_lds(S.kt + (md * 16 + (lane & 15)) * LDT, S.t2 + (nt * 16 + (lane & 15)) * LDT,
                            nt + 1, g, zero4());
    store4_h(S.kr + (nt * 16 + (lane & 15)) * L::LDK + md * 16 + 4 * g, -w[0], -w[1], -w[2], -w[3]);
  }
}

// Common per-sub-chunk preparation: write the staged sub-chunk to LDS, start
// fetching the next one (if any), then Gram, Tm and -W.
template <int D, bool OUT>
__device__ __forceinline__ void prepare(const Args& a, const Smem<D, OUT>& S, Stage& st, int b, int h,
                                        bool has_next, long long t0n, int nn, bool rev) {
  const int wave = wave_id();
  __syncthreads();
  stage_subchunk<D, OUT>(S, st);
  if (has_next) fetch_subchunk<D, OUT>(a, b, h, t0n, nn, rev, st);
  __syncthreads();
  gram_stage<D, OUT>(a, S);
  __syncthreads();
  if (wave == 0) diag_inverse<D, OUT>(a, S);
  __syncthreads();
  offdiag_inverse<D, OUT>(a, S);
  __syncthreads();
  w_stage<D, OUT>(S);
}

// Per-lane row factors of token tile mt (rows 16 mt + 4 g + r):
// exp(G_i) and c exp(G_n - G_i).
__device__ __forceinline__ f32x4 row_decay(const float* g2, int mt, int g) {
  const float4 v = *reinterpret_cast<const float4*>(g2 + mt * 16 + 4 * g);
  return f32x4{exp2f(v.x), exp2f(v.y), exp2f(v.z), exp2f(v.w)};
}
__device__ __forceinline__ f32x4 row_scale(const float* g2, float glast, float c, int mt, int g) {
  const float4 v = *reinterpret_cast<const float4*>(g2 + mt * 16 + 4 * g);
  return f32x4{c * exp2f(glast - v.x), c * exp2f(glast - v.y), c * exp2f(glast - v.z), c * exp2f(glast - v.w)};
}

// ---------------------------------------------------------------------------
// 1. Segment maps.  grid (NS - 1, B * H, ndir).  The state X = [P | Q]
// (D x 2D) is split into 16-column strips; wavefront w owns strips w, w + NW, ...
template <int D>
__global__ __launch_bounds__(NT) void seg_map_kernel(Args a) {
  using L = Lay<D, false>;
  constexpr int MD = D / 16, NS_ = 2 * MD, SPW = (NS_ + NW - 1) / NW;
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
  const Smem<D, false> S(smem);
  const int wave = wave_id(), lane = threadIdx.x & 63, g = lane >> 4, cl = lane & 15;
  const int pos = blockIdx.x;                       // scan position of the segment
  const int bh_ = blockIdx.y, b = bh_ / a.H, h = bh_ % a.H;
  const int slot = blockIdx.z, dir = dir_of_slot(a.dirs, slot);
  const bool rev = dir == 1;
  const int seg = rev ? a.NS - 1 - pos : pos;
  const long long s0 = (long long)seg * a.L;
  const long long s1 = (s0 + a.L < a.T) ? s0 + a.L : a.T;
  const int nsub = (int)((s1 - s0 + CH - 1) / CH);

  for (int i = threadIdx.x; i < 4 * CH * LDT / 2; i += NT) reinterpret_cast<uint32_t*>(S.ab)[i] = 0u;

  f32x4 X[SPW][MD];
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int st = wave + NW * j;
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int r = 0; r < 4; ++r) X[j][md][r] = (st == md && 4 * g + r == cl) ? 1.f : 0.f;
  }

  // sub-chunk jj of the scan: its first original token and size
  auto piece = [&](int jj, long long& t0, int& n) {
    const int jc = rev ? nsub - 1 - jj : jj;
    t0 = s0 + (long long)jc * CH;
    n = (int)((s1 - t0) < CH ? (s1 - t0) : CH);
  };
  Stage st;
  {
    long long t0;
    int n;
    piece(0, t0, n);
    fetch_subchunk<D, false>(a, b, h, t0, n, rev, st);
  }
  for (int jj = 0; jj < nsub; ++jj) {
    long long t0, t0n = 0;
    int n, nn = 0;
    piece(jj, t0, n);
    if (jj + 1 < nsub) piece(jj + 1, t0n, nn);
    prepare<D, false>(a, S, st, b, h, jj + 1 < nsub, t0n, nn, rev);
    // U strips (values part only)
    f32x4 V[SPW][4];
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int st = wave + NW * j;
      const int vs = st < MD ? 0 : (st < NS_ ? st - MD : MD - 1);   // value strip (clamped)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f32x4 u = mma_lds(S.t1 + (mt * 16 + cl) * LDT, S.vt + (vs * 16 + cl) * LDT, mt + 1, g, zero4());
        V[j][mt] = st >= MD ? u : zero4();          // the P part has no values
      }
    }
    __syncthreads();
    const float glast = S.g2[CH - 1];
    const float dec = exp2f(glast);
    // fp16 copy of the state as MFMA B pairs (rows = d)
    f16x8_t Xp[SPW][MD / 2 > 0 ? MD / 2 : 1];
    f16x4_t Xq[SPW];
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
#pragma unroll
      for (int p = 0; p < MD / 2; ++p) Xp[j][p] = tof16x8(X[j][2 * p], X[j][2 * p + 1]);
      if constexpr (MD & 1) Xq[j] = tof16(X[j][MD - 1]);
    }
    // V'aug = [0 | U] - W X   (per token tile mt, all strips at once)
    f32x4 Vf[SPW][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 acc[SPW];
#pragma unroll
      for (int j = 0; j < SPW; ++j) acc[j] = V[j][mt];
      mma_dB<SPW, MD / 2, (MD & 1) != 0>(S.kr + (mt * 16 + cl) * L::LDK, Xp, Xq, g, acc);
      const f32x4 sc = row_scale(S.g2, glast, a.c, mt, g);
#pragma unroll
      for (int j = 0; j < SPW; ++j) Vf[j][mt] = acc[j] * sc;
    }
    f16x8_t Vs[SPW][2];
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      Vs[j][0] = tof16x8(Vf[j][0], Vf[j][1]);
      Vs[j][1] = tof16x8(Vf[j][2], Vf[j][3]);
    }
    // X <- e^{G_n} X + c K^T diag(e^{G_n - G}) V'aug
#pragma unroll
    for (int md = 0; md < MD; ++md) {
      f32x4 acc[SPW];
#pragma unroll
      for (int j = 0; j < SPW; ++j) acc[j] = X[j][md] * dec;
      mma_tB<SPW>(S.kt + (md * 16 + cl) * LDT, Vs, 4, g, acc);
#pragma unroll
      for (int j = 0; j < SPW; ++j) X[j][md] = acc[j];
    }
  }
  // store X = [P | Q] (fp32, row-major [D][2D])
  float* Xg = a.maps + ((((size_t)slot * a.B + b) * a.H + h) * (a.NS - 1) + pos) * (size_t)D * (2 * D);
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int st = wave + NW * j;
    if (st < NS_) {
#pragma unroll
      for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int r = 0; r < 4; ++r) Xg[(size_t)(md * 16 + 4 * g + r) * (2 * D) + st * 16 + cl] = X[j][md][r];
    }
  }
}

// ---------------------------------------------------------------------------
// 2. Segment chain.  grid (DV / 16, B * H, ndir).  H_{p+1} = P_p H_p + Q_p on
// one 16-column tile of the state, fp32 carried in registers; products in
// split bf16 (x = hi + lo, hi*hi + hi*lo + lo*hi).
template <int D>
__global__ __launch_bounds__(NTC) void seg_chain_kernel(Args a) {
  constexpr int DK = D, DV = D;
  constexpr int MD = DK / 16, LDK = DK + 8, NXC = DK + DV;
  constexpr int MSLOTS = (MD + NWC - 1) / NWC;
  __shared__ __attribute__((aligned(16))) bh hhi[16 * LDK];
  __shared__ __attribute__((aligned(16))) bh hlo[16 * LDK];
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int nv = blockIdx.x;
  const int bh_ = blockIdx.y, b = bh_ / a.H, h = bh_ % a.H;
  const int slot = blockIdx.z, dir = dir_of_slot(a.dirs, slot);
  const float* seed = (dir == 0 || a.dirs == 2) ? a.h0 : nullptr;
  const int col = nv * 16 + (lane & 15);
  const size_t sbase = ((size_t)b * a.H + h) * DK * DV;

  f32x4 hs[MSLOTS];
#pragma unroll
  for (int s = 0; s < MSLOTS; ++s) {
    const int md = wave + NWC * s;
    const int row0 = md * 16 + 4 * (lane >> 4);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      hs[s][r] = (md < MD && seed) ? seed[sbase + (size_t)(row0 + r) * DV + col] : 0.f;
  }
  float* st = a.starts + (((size_t)slot * a.B + b) * a.H + h) * (size_t)a.NS * DK * DV;
  for (int p = 0;; ++p) {
    // record the start state of segment p and publish H for the product
#pragma unroll
    for (int s = 0; s < MSLOTS; ++s) {
      const int md = wave + NWC * s;
      if (md < MD) {
        const int row0 = md * 16 + 4 * (lane >> 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) st[(size_t)p * DK * DV + (size_t)(row0 + r) * DV + col] = hs[s][r];
        uint2 uh, ul;
        bh hh[4], hl[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          hh[r] = f2bh(hs[s][r]);
          hl[r] = f2bh(hs[s][r] - bh2f(hh[r]));
        }
        uh.x = hh[0] | ((uint32_t)hh[1] << 16);
        uh.y = hh[2] | ((uint32_t)hh[3] << 16);
        ul.x = hl[0] | ((uint32_t)hl[1] << 16);
        ul.y = hl[2] | ((uint32_t)hl[3] << 16);
        *reinterpret_cast<uint2*>(hhi + (lane & 15) * LDK + row0) = uh;
        *reinterpret_cast<uint2*>(hlo + (lane & 15) * LDK + row0) = ul;
      }
    }
    if (p == a.NS - 1) break;
    __syncthreads();
    const float* X = a.maps + ((((size_t)slot * a.B + b) * a.H + h) * (a.NS - 1) + p) * (size_t)DK * NXC;
#pragma unroll
    for (int s = 0; s < MSLOTS; ++s) {
      const int md = wave + NWC * s;
      if (md < MD) {
        const int row0 = md * 16 + 4 * (lane >> 4);
        f32x4 acc;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = X[(size_t)(row0 + r) * NXC + DK + col];
        const float* prow = X + (size_t)(md * 16 + (lane & 15)) * NXC;
        const int g = lane >> 4;
        int k = 0;
#pragma unroll
        for (; k + 32 <= DK; k += 32) {
          const float4 v0 = *reinterpret_cast<const float4*>(prow + k + 8 * g);
          const float4 v1 = *reinterpret_cast<const float4*>(prow + k + 8 * g + 4);
          const float pv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
          bf16x8_t ahi, alo;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const __bf16 hi = static_cast<__bf16>(pv[e]);
            ahi[e] = hi;
            alo[e] = static_cast<__bf16>(pv[e] - static_cast<float>(hi));
          }
          const bf16x8_t bhi = *reinterpret_cast<const bf16x8_t*>(hhi + (lane & 15) * LDK + k + 8 * g);
          const bf16x8_t blo = *reinterpret_cast<const bf16x8_t*>(hlo + (lane & 15) * LDK + k + 8 * g);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bhi, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, blo, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bhi, acc, 0, 0, 0);
        }
        if constexpr ((DK % 32) != 0) {
          const float4 v0 = *reinterpret_cast<const float4*>(prow + k + 4 * g);
          const float pv[4] = {v0.x, v0.y, v0.z, v0.w};
          s16x4_t ahi, alo;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bh hi = f2bh(pv[e]);
            ahi[e] = (short)hi;
            alo[e] = (short)f2bh(pv[e] - bh2f(hi));
          }
          const s16x4_t bhi = *reinterpret_cast<const s16x4_t*>(hhi + (lane & 15) * LDK + k + 4 * g);
          const s16x4_t blo = *reinterpret_cast<const s16x4_t*>(hlo + (lane & 15) * LDK + k + 4 * g);
          // K = 16 tail in its own accumulator (one MFMA shape per chain)
          f32x4 tail = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ahi, bhi, zero4(), 0, 0, 0);
          tail = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ahi, blo, tail, 0, 0, 0);
          tail = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(alo, bhi, tail, 0, 0, 0);
          acc = acc + tail;
        }
        hs[s] = acc;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// 3. Outputs.  grid (NS, B * H).  Each workgroup runs its segment for every
// requested direction (reversed scan first) from the start states of the
// chain; the reversed scan's outputs are summed into the forward scan's.
// Wavefront w owns the state's 16-column strips w, w + NW, ...
template <int D>
__global__ __launch_bounds__(NT) void seg_out_kernel(Args a) {
  using L = Lay<D, true>;
  constexpr int MD = D / 16, SPW = (MD + NW - 1) / NW;
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
  const Smem<D, true> S(smem);
  const int wave = wave_id(), lane = threadIdx.x & 63, g = lane >> 4, cl = lane & 15;
  const int seg = blockIdx.x;
  const int bh_ = blockIdx.y, b = bh_ / a.H, h = bh_ % a.H;
  const long long s0 = (long long)seg * a.L;
  const long long s1 = (s0 + a.L < a.T) ? s0 + a.L : a.T;
  const int nsub = (int)((s1 - s0 + CH - 1) / CH);
  const size_t sbase = ((size_t)b * a.H + h) * D * D;

  for (int i = threadIdx.x; i < 5 * CH * LDT / 2; i += NT) reinterpret_cast<uint32_t*>(S.ab)[i] = 0u;

  for (int pass = 0; pass < 2; ++pass) {
    const int dir = pass == 0 ? 1 : 0;                 // reversed scan first
    if (!(a.dirs & (1 << dir))) continue;
    const bool rev = dir == 1;
    const int mode = a.dirs == 3 ? (rev ? 1 : 2) : 0;   // 1: write partial, 2: add partial
    const int slot = slot_of_dir(a.dirs, dir);
    const int pos = rev ? a.NS - 1 - seg : seg;
    const float* stp = a.starts + ((((size_t)slot * a.B + b) * a.H + h) * a.NS + pos) * (size_t)D * D;
    f32x4 H[SPW][MD];
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int st = wave + NW * j;
#pragma unroll
      for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int r = 0; r < 4; ++r) H[j][md][r] = (st < MD) ? stp[(size_t)(md * 16 + 4 * g + r) * D + st * 16 + cl] : 0.f;
    }
    auto piece = [&](int jj, long long& t0, int& n) {
      const int jc = rev ? nsub - 1 - jj : jj;
      t0 = s0 + (long long)jc * CH;
      n = (int)((s1 - t0) < CH ? (s1 - t0) : CH);
    };
    Stage st;
    {
      long long t0;
      int n;
      piece(0, t0, n);
      fetch_subchunk<D, true>(a, b, h, t0, n, rev, st);
    }
    for (int jj = 0; jj < nsub; ++jj) {
      long long t0, t0n = 0;
      int n, nn = 0;
      piece(jj, t0, n);
      if (jj + 1 < nsub) piece(jj + 1, t0n, nn);
      prepare<D, true>(a, S, st, b, h, jj + 1 < nsub, t0n, nn, rev);
      f32x4 V[SPW][4];
#pragma unroll
      for (int j = 0; j < SPW; ++j) {
        const int st = wave + NW * j;
        const int vs = st < MD ? st : MD - 1;      // clamped strip
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          V[j][mt] = mma_lds(S.t1 + (mt * 16 + cl) * LDT, S.vt + (vs * 16 + cl) * LDT, mt + 1, g, zero4());
      }
      __syncthreads();
      const float glast = S.g2[CH - 1];
      const float dec = exp2f(glast);
      f16x8_t Hp[SPW][MD / 2 > 0 ? MD / 2 : 1];
      f16x4_t Hq[SPW];
#pragma unroll
      for (int j = 0; j < SPW; ++j) {
#pragma unroll
        for (int p = 0; p < MD / 2; ++p) Hp[j][p] = tof16x8(H[j][2 * p], H[j][2 * p + 1]);
        if constexpr (MD & 1) Hq[j] = tof16(H[j][MD - 1]);
      }
      // V' = U - W H
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4 acc[SPW];
#pragma unroll
        for (int j = 0; j < SPW; ++j) acc[j] = V[j][mt];
        mma_dB<SPW, MD / 2, (MD & 1) != 0>(S.kr + (mt * 16 + cl) * L::LDK, Hp, Hq, g, acc);
#pragma unroll
        for (int j = 0; j < SPW; ++j) V[j][mt] = acc[j];
      }
      f16x8_t Vh[SPW][2], Vs[SPW][2];
#pragma unroll
      for (int j = 0; j < SPW; ++j) {
        Vh[j][0] = tof16x8(V[j][0], V[j][1]);
        Vh[j][1] = tof16x8(V[j][2], V[j][3]);
        const f32x4 s0 = row_scale(S.g2, glast, a.c, 0, g), s1 = row_scale(S.g2, glast, a.c, 1, g);
        const f32x4 s2 = row_scale(S.g2, glast, a.c, 2, g), s3 = row_scale(S.g2, glast, a.c, 3, g);
        Vs[j][0] = tof16x8(V[j][0] * s0, V[j][1] * s1);
        Vs[j][1] = tof16x8(V[j][2] * s2, V[j][3] * s3);
      }
      // O = diag(e^G) Q H + P V'
      const long long tstride = rev ? -(long long)a.H * D : (long long)a.H * D;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4 acc[SPW];
#pragma unroll
        for (int j = 0; j < SPW; ++j) acc[j] = zero4();
        mma_dB<SPW, MD / 2, (MD & 1) != 0>(S.qr + (mt * 16 + cl) * L::LDK, Hp, Hq, g, acc);
        const f32x4 eg = row_decay(S.g2, mt, g);
#pragma unroll
        for (int j = 0; j < SPW; ++j) acc[j] = acc[j] * eg;
        mma_tB<SPW>(S.p + (mt * 16 + cl) * LDT, Vh, mt + 1, g, acc);
        const int i0 = mt * 16 + 4 * g;                       // scan-local row of r = 0
        const size_t e0 = ((size_t)b * a.T + token_of(t0, n, rev, i0)) * a.H * D + (size_t)h * D;
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
          const int st = wave + NW * j;
          if (st < MD) {
            const size_t base = e0 + st * 16 + cl;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              if (i0 + r < n) {
                const size_t off = base + r * tstride;
                float val = acc[j][r];
                if (mode == 1) {
                  a.acc[off] = val;
                } else {
                  if (mode == 2) val += a.acc[off];
                  if (a.out_bf16) static_cast<uint16_t*>(a.out)[off] = f32_to_bf16_bits(val);
                  else static_cast<float*>(a.out)[off] = val;
                }
              }
            }
          }
        }
      }
      // H <- e^{G_n} H + c K^T diag(e^{G_n - G}) V'
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        f32x4 acc[SPW];
#pragma unroll
        for (int j = 0; j < SPW; ++j) acc[j] = H[j][md] * dec;
        mma_tB<SPW>(S.kt + (md * 16 + cl) * LDT, Vs, 4, g, acc);
#pragma unroll
        for (int j = 0; j < SPW; ++j) H[j][md] = acc[j];
      }
    }
    // final state: the scan's last segment
    if (a.hT && pos == a.NS - 1 && (dir == 0 || a.dirs == 2)) {
#pragma unroll
      for (int j = 0; j < SPW; ++j) {
        const int st = wave + NW * j;
        if (st < MD) {
#pragma unroll
          for (int md = 0; md < MD; ++md)
#pragma unroll
            for (int r = 0; r < 4; ++r) a.hT[sbase + (size_t)(md * 16 + 4 * g + r) * D + st * 16 + cl] = H[j][md][r];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
struct Plan {
  int L, NS, ndir, dirs;
  size_t maps_off, starts_off, acc_off, bytes;
};

Plan make_plan(const Problem& p, int direction) {
  Plan pl{};
  pl.dirs = direction == GDN_FORWARD ? 1 : direction == GDN_BACKWARD ? 2 : 3;
  pl.ndir = pl.dirs == 3 ? 2 : 1;
  int L = g_segment_override.load(std::memory_order_relaxed);
  if (L <= 0) {
    // enough segments for ~2048 output workgroups
    const long long hb = (long long)p.B * p.H;
    const long long want = (2048 + hb - 1) / hb;
    long long per = (p.T + want - 1) / want;
    L = (int)((per + CH - 1) / CH * CH);
  }
  L = (L + CH - 1) / CH * CH;
  if (L < CH) L = CH;
  if ((long long)L > p.T) L = (int)((p.T + CH - 1) / CH * CH);
  pl.L = L;
  pl.NS = (int)((p.T + L - 1) / L);
  const size_t bhd = (size_t)pl.ndir * p.B * p.H;
  const size_t maps = bhd * (size_t)(pl.NS - 1) * p.dk * (p.dk + p.dv) * sizeof(float);
  const size_t starts = bhd * (size_t)pl.NS * p.dk * p.dv * sizeof(float);
  const size_t acc = (pl.dirs == 3 && p.out_bf16) ? (size_t)p.B * p.T * p.H * p.dv * sizeof(float) : 0;
  pl.maps_off = 0;
  pl.starts_off = align_up(maps, 256);
  pl.acc_off = pl.starts_off + align_up(starts, 256);
  pl.bytes = pl.acc_off + align_up(acc, 256);
  return pl;
}

template <int D>
hipError_t launch_d(const Problem& p, const Plan& pl, const Tensors& t, char* ws, hipStream_t stream) {
  Args a{};
  a.q = static_cast<const bh*>(t.q);
  a.k = static_cast<const bh*>(t.k);
  a.v = static_cast<const bh*>(t.v);
  a.g = t.g;
  a.beta = t.beta;
  a.h0 = t.h0;
  a.out = t.out;
  a.hT = t.hT;
  a.maps = reinterpret_cast<float*>(ws + pl.maps_off);
  a.starts = reinterpret_cast<float*>(ws + pl.starts_off);
  a.acc = p.out_bf16 ? reinterpret_cast<float*>(ws + pl.acc_off) : static_cast<float*>(t.out);
  a.T = p.T;
  a.B = p.B;
  a.H = p.H;
  a.L = pl.L;
  a.NS = pl.NS;
  a.dirs = pl.dirs;
  a.out_bf16 = p.out_bf16 ? 1 : 0;
  a.c = p.key_scale;
  const unsigned bhc = (unsigned)(p.B * p.H);
  if (pl.NS > 1) {
    prof_begin(stream, GDN_KERNEL_SEG_MAP);
    hipLaunchKernelGGL((seg_map_kernel<D>), dim3(pl.NS - 1, bhc, pl.ndir), dim3(NT), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    prof_end(stream, GDN_KERNEL_SEG_MAP);
  }
  prof_begin(stream, GDN_KERNEL_SEG_CHAIN);
  hipLaunchKernelGGL((seg_chain_kernel<D>), dim3(D / 16, bhc, pl.ndir), dim3(NTC), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof_end(stream, GDN_KERNEL_SEG_CHAIN);
  prof_begin(stream, GDN_KERNEL_SEG_OUT);
  hipLaunchKernelGGL((seg_out_kernel<D>), dim3(pl.NS, bhc, 1), dim3(NT), 0, stream, a);
  e = hipGetLastError();
  prof_end(stream, GDN_KERNEL_SEG_OUT);
  return e;
}

}  // namespace

const char* chunked_unsupported_reason(const Problem& p) {
  if (!p.qkv_bf16) return "q, k and v must be bf16";
  if (p.dk != p.dv) return "d_k must equal d_v";
  if (p.dk > 112) return "d_k = d_v must be at most 112";
  if (p.B * (long long)p.H > 65535) return "batch * heads must be at most 65535";
  const Plan pl = make_plan(p, GDN_FORWARD);
  if (pl.NS > 2147483647 / 2) return "too many segments";
  return nullptr;
}

size_t chunked_workspace(const Problem& p, int direction) { return make_plan(p, direction).bytes; }

hipError_t chunked_launch(const Problem& p, int direction, const Tensors& t, void* workspace,
                          hipStream_t stream) {
  const Plan pl = make_plan(p, direction);
  char* ws = static_cast<char*>(workspace);
  switch (p.dk) {
    case 16: return launch_d<16>(p, pl, t, ws, stream);
    case 32: return launch_d<32>(p, pl, t, ws, stream);
    case 48: return launch_d<48>(p, pl, t, ws, stream);
    case 64: return launch_d<64>(p, pl, t, ws, stream);
    case 80: return launch_d<80>(p, pl, t, ws, stream);
    case 96: return launch_d<96>(p, pl, t, ws, stream);
    case 112: return launch_d<112>(p, pl, t, ws, stream);
    default: return hipErrorInvalidValue;
  }
}

int chunked_segment_tokens(const Problem& p, int direction) { return make_plan(p, direction).L; }

void set_segment_tokens(int tokens) { g_segment_override.store(tokens > 0 ? tokens : 0); }

}  // namespace gdn
