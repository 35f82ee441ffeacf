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
//     R   = V - c diag(e^G) K H              (values minus the decayed prediction)
//     V'  = Tm diag(beta) R                  (the per-token corrections)
//     O   = diag(e^G) Q H + (c tril(Q K^T) * E) V'       (read after write)
//     H  <- e^{G_n} H + c K^T diag(e^{G_n - G}) V'
// (V' equals the WY/UT form U - W H with U = Tm diag(beta) V and
// W = c Tm diag(beta e^G) K; the R form needs neither W nor U.)
//
// Schedule.  The token axis is cut, in original order, into segments of L
// tokens (a multiple of 64) and each segment into 64-token sub-chunks; a scan
// direction visits both in its own order.  Per scan direction:
//   1. seg_map_kernel   (parallel over segments): the segment's affine state
//      map H_end = P H_start + Q, by running the sub-chunk chain on the
//      augmented state X = [P | Q] from [I | 0] with values [0 | V]
//      (seg_map_q_kernel: Q alone, for the reversed scan of a bidirectional
//      call, whose P is the transpose of the forward one);
//   2. seg_chain_kernel (serial over segments, parallel over heads and value
//      columns): H_{s+1} = P_s H_s + Q_s in split-bf16 (hi + lo) MFMA, i.e. the
//      prefix composition of the segments' transition maps, whole or split
//      into groups (compose, chain of groups, expand);
//   3. seg_out_kernel   (parallel over segments): each segment re-run from its
//      true start state, writing outputs and the final state.  In a
//      bidirectional call the forward launch stores an fp16 partial and the
//      reversed launch adds it before the single final store.
// The frame-level (Jacobi) transition at the end of this file reuses the
// chain kernel between its own per-frame map and output kernels.
//
// Workgroups of the map and output kernels: one wavefront per 16-column strip
// of the state ("strip waves", the state strip lives in its registers) plus
// one helper wavefront.  Per sub-chunk c there are two phases:
//   alpha: the strip waves write their share of sub-chunk c+1's rows into the
//          other LDS buffer (and store c-1's outputs) and form K H and R; the
//          helper stages c+1's gate factors and inverts the off-diagonal
//          blocks of I + A_c.
//   beta:  the strip waves form Q H, V', the outputs and the new state and
//          the off-diagonal Gram tiles (A and P) of sub-chunk c+1; the helper
//          forms and inverts c+1's diagonal blocks.
// so the triangular inverse, which is serial, overlaps the state products.
// All states and accumulations are fp32.  MFMA operands are fp16: the bf16
// inputs convert to fp16 exactly (in fp16's normal range) and each rounded
// intermediate (Tm, H, R, V', P) keeps 11 significant bits.  Precondition of
// this path: inputs and intermediate magnitudes stay below fp16's maximum
// (65504).  The map and output kernels use the 16x16x32 f16 MFMA (16x16x16
// for the inverse's block products, from a zero accumulator); the chain uses
// the 16x16x32 bf16 form on split operands.
#include "gdn_common.h"
#include "gdn_internal.h"
#include "gdn_mfma.h"

#include <mutex>

namespace gdn {
namespace {

constexpr int CH = 64;          // sub-chunk tokens
constexpr int LDT = CH + 8;     // row stride (elements) of token-contracted fp16 matrices
constexpr int LDD = 24;         // row stride of the diagonal inverse blocks
constexpr int ADB = 260;        // float stride of the fp32 diagonal blocks of A (16 x 16 + pad)
constexpr float kLog2e = 1.4426950408889634f;

// Maps per group of a split chain for `nsteps` steps, or 0 for the whole chain
// in one pass.  k: the problem's chain_group (0 automatic: split chains of 16
// steps or more into groups of ceil(sqrt(nsteps / 2)) maps, whose serial steps
// 2m + G are minimal near that m).
int chain_group(int nsteps, int k) {
  if (k == 1) return 0;
  if (k >= 2) return nsteps > k ? k : 0;
  if (nsteps < 16) return 0;
  int m = 1;
  while (2 * m * m < nsteps) ++m;
  return m;
}

// Workspace of a (possibly split) chain: group maps and group start states.
struct ChainWs {
  int m = 0, groups = 0;
  size_t gmaps_bytes = 0, gstarts_bytes = 0;
};
ChainWs chain_ws(int nsteps, int k, size_t heads_dirs, int dk, int dv) {
  ChainWs c;
  c.m = chain_group(nsteps, k);
  if (c.m > 0) {
    c.groups = (nsteps + c.m - 1) / c.m;
    c.gmaps_bytes = align_up(heads_dirs * c.groups * (size_t)dk * (dk + dv) * sizeof(float), 256);
    c.gstarts_bytes = align_up(heads_dirs * c.groups * (size_t)dk * dv * sizeof(float), 256);
  }
  return c;
}

struct Args {
  const bh* q;
  const bh* k;
  const bh* v;
  const float* g;
  const float* beta;
  const float* h0;      // initial state or null
  void* out;
  hb* part;             // fp16 partial outputs of the first output launch of a two-scan call
  float* hT;            // final state or null
  float* maps;          // [ndir][B][H][NS][DK][DK+DV]
  float* starts;        // [ndir][B][H][NS][DK][DV]
  long long T;
  int B, H, L, NS;
  int dirs;             // bit 0: forward scan, bit 1: reversed scan
  int slot0;            // map and chain kernels: slot of blockIdx direction index 0
  int heads_rev;        // map and output kernels: visit the (batch, head) pairs in reversed order
  int npos;             // map and output kernels: segments in the launch (gridDim.x may be larger)
  long long cs_first;   // output kernel, chunk-causal reversed scan: tokens of the first chunk
  long long cs_len;     // ... and of every later chunk (0: segments of L tokens from the chain)
  int dir;              // output kernel: the scan direction of this launch (1: reversed)
  int mode;             // output kernel: 0 store outputs, 1 store the partial, 2 add the partial
  int out_bf16;
  float c;              // key scale
  const float* fac;     // feature prologue factors (fk, fq) per token, [B][H][T + 2][2] (token t at t + 1), or null
  int ch_mode;          // chain kernel: 0 whole chain, 1 compose groups, 2 chain of groups, 3 expand groups
  int ch_m, ch_groups;  // ... maps per group, groups
  float* gmaps;         // ... composed group maps [ndir][B][H][groups][DK][DK+DV]
  float* gstarts;       // ... group start states [ndir][B][H][groups][DK][DV] (transposed)
  char* sc;             // strip scan: per sub-chunk and head, Tm diag(beta), P and gate factors
  hb* tm;               // Tm diag(beta) of every sub-chunk, [ndir][B][H][U][10][16][16] (U = ceil(T / 64),
                        // the 10 lower 16x16 blocks), stored by the map kernels and read by the output
                        // kernels; null: the map kernels store nothing
};

// Wavefront index as a wave-uniform (scalar) value, so that branches on it are
// scalar branches rather than per-lane exec masking.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ int dir_of_slot(int dirs, int slot) {
  // slot 0 is the forward scan when present
  return (dirs & 1) ? (slot == 0 ? 0 : 1) : 1;
}
__device__ __forceinline__ int slot_of_dir(int dirs, int dir) { return (dir == 1 && (dirs & 1)) ? 1 : 0; }

// Workgroup geometry for state width D.
template <int D>
struct Geo {
  static constexpr int MD = D / 16;              // 16-wide tiles along d
  static constexpr int NSW = MD;                 // strip wavefronts
  static constexpr int HW = NSW;                 // index of the helper wavefront
  static constexpr int NT = 64 * (NSW + 1);      // threads per workgroup
  static constexpr int DP = (D + 31) / 32 * 32;  // d padded to whole K = 32 steps
  static constexpr int NP = DP / 32;
  // Row stride (elements) of the staged V rows: at least D and = 16 (mod 32),
  // i.e. an odd multiple of 8 words, so that the 8 consecutive rows x 32 bytes
  // of a transposing read per half wavefront fall on distinct banks.
  static constexpr int LDV = (D + 15) / 32 * 32 + 16;
};

// K and Q rows (fp16, d-contracted): row r starts at r LDK + 8 (r / 8)
// elements, with LDK = D (D = 16 mod 32) or D + 16 (D = 0 mod 32).  In units of
// 8 bytes, LDK / 4 is then 4 times an odd number, so the starts of 8
// consecutive rows fall on distinct multiples of 4 banks (mod 32 units), and
// the 16-byte step every 8 rows puts rows 8..15 of a 16-row block on the
// remaining even offsets.  Both ways these rows are read are then free of bank
// conflicts per half wavefront: 16 consecutive rows x 2 adjacent 8-byte units
// (fragment reads), and 8 consecutive rows x 4 adjacent units (transposing
// reads of K^T).  krow is additive over a multiple-of-8 row offset, so every
// read is a per-lane base plus an immediate.
template <int D>
struct KRows {
  static constexpr int LDK = D % 32 == 0 ? D + 16 : D;
  static constexpr int ELEMS = CH * LDK + 8 * (CH / 8);
};
template <int D>
__device__ __forceinline__ constexpr int krow(int r) { return r * KRows<D>::LDK + 8 * (r >> 3); }

// Shared memory.  Two sub-chunk buffers (Q and K rows, P, the inverse, gate
// factors) alternate between "being computed on" and "being prepared"; the V
// rows (read in phase alpha only, so the next ones are written in beta), the A
// matrix, the helper's diagonal blocks and the output staging rows are
// single-buffered (their producer and consumer phases are separated by a
// barrier).  OUT: output pass (else map pass: no Q, no P, no outputs).
template <int D, bool OUT>
struct Lay {
  using G = Geo<D>;
  static constexpr int QR = OUT ? (KRows<D>::ELEMS * 2 + 15) / 16 * 16 : 0;
  static constexpr int KR = (KRows<D>::ELEMS * 2 + 15) / 16 * 16;
  static constexpr int VR = CH * G::LDV * 2;
  static constexpr int PP = OUT ? CH * LDT * 2 : 0;
  static constexpr int TT = CH * LDT * 2;
  static constexpr int GT = 5 * CH * 4;
  static constexpr int o_qr = 0;
  static constexpr int o_kr = o_qr + QR;
  static constexpr int o_pp = o_kr + KR;
  static constexpr int o_tt = o_pp + PP;               // Tm diag(beta), fp16 rows
  static constexpr int o_gt = o_tt + TT;
  static constexpr int BUF = o_gt + GT;
  static constexpr int o_vr = 2 * BUF;                 // V rows, raw bf16
  // output staging: 64 rows of D fp32 values, OSL floats apart (D + 4: the
  // 16-row columns of a tile write fall on distinct banks)
  static constexpr int OSL = D + 4;
  static constexpr int OS = OUT ? CH * OSL * 4 : 0;
  static constexpr int o_os = o_vr + VR;
  static constexpr int o_ao = o_os + OS;               // off-diagonal blocks of A, fp16 rows
  static constexpr int o_td = o_ao + CH * LDT * 2;     // diagonal blocks of Tm, fp16 rows
  static constexpr int o_ad = o_td + CH * LDD * 2;     // diagonal blocks of A, fp32
  static constexpr int BYTES = o_ad + 4 * ADB * 4;
  static_assert(BYTES <= 160 * 1024, "workgroup LDS budget exceeded");
  static_assert(QR % 16 == 0 && KR % 16 == 0 && VR % 16 == 0 && PP % 16 == 0 && BUF % 16 == 0, "alignment");
};

// One sub-chunk buffer.
struct Buf {
  hb *qr, *kr, *pp, *tt;
  bh* vr;
  float *g2, *eg, *ce, *dn, *bt;   // cumsum (log2), e^G, c e^G, c e^{G_n - G}, beta
};

// An LDS base address the compiler must treat as computed here: every LDS
// address of the loop body is then this base plus an immediate offset, instead
// of one loop-invariant address register per array and lane pattern (which the
// compiler would otherwise hoist and keep live for the whole kernel).
__device__ __forceinline__ char* lds_at(char* smem, uint32_t off) {
  asm volatile("" : "+v"(off));
  return smem + off;
}

template <int D, bool OUT>
__device__ __forceinline__ Buf buf_at(char* s, int i) {
  using L = Lay<D, OUT>;
  char* p = lds_at(s, (uint32_t)(i * L::BUF));
  Buf b;
  b.qr = reinterpret_cast<hb*>(p + L::o_qr);
  b.kr = reinterpret_cast<hb*>(p + L::o_kr);
  b.vr = reinterpret_cast<bh*>(lds_at(s, (uint32_t)L::o_vr));
  b.pp = reinterpret_cast<hb*>(p + L::o_pp);
  b.tt = reinterpret_cast<hb*>(p + L::o_tt);
  float* gt = reinterpret_cast<float*>(p + L::o_gt);
  b.g2 = gt;
  b.eg = gt + CH;
  b.ce = gt + 2 * CH;
  b.dn = gt + 3 * CH;
  b.bt = gt + 4 * CH;
  return b;
}

// Single-buffered arrays of the inverse.
struct Inv {
  hb *ao, *td;
  float* ad;
  float* os;   // output staging rows (output pass)
};

template <int D, bool OUT>
__device__ __forceinline__ Inv inv_at(char* s0) {
  using L = Lay<D, OUT>;
  char* s = lds_at(s0, 0u);
  Inv v;
  v.ao = reinterpret_cast<hb*>(s + L::o_ao);
  v.td = reinterpret_cast<hb*>(s + L::o_td);
  v.ad = reinterpret_cast<float*>(s + L::o_ad);
  v.os = reinterpret_cast<float*>(s + L::o_os);
  return v;
}

__device__ __forceinline__ void store4_h(hb* dst, float a, float b, float c, float d) {
  uint2 u;
  u.x = static_cast<uint32_t>(f2h(a)) | (static_cast<uint32_t>(f2h(b)) << 16);
  u.y = static_cast<uint32_t>(f2h(c)) | (static_cast<uint32_t>(f2h(d)) << 16);
  *reinterpret_cast<uint2*>(dst) = u;
}

// --- MFMA helpers -------------------------------------------------------------
// A 16x16 accumulator tile X (lane l: X[4(l/16) + r][l % 16]) converted to
// fp16 is directly the B operand of a 16x16x16 product contracting over X's
// rows.  Two such tiles (rows 0-15 and 16-31 of the contraction) form the B
// operand of a 16x16x32 product whose k order is {4g..4g+3, 16+4g..16+4g+3}
// for lane group g; the A operand is then read from LDS in that same order.

// Fragment halves are read with one ds_read_b64 each.  The loads are volatile
// only so that the compiler does not pair them into ds_read2_b64: measured on
// gfx950, a 16-row fragment read as two ds_read_b64 occupies the LDS for 4
// cycles, the same data as one ds_read2_b64 for 16 (bank conflicts).
typedef __attribute__((address_space(3))) const volatile f16x4_t lds_f16x4_t;
__device__ __forceinline__ f16x4_t ld4(const hb* p) { return *(lds_f16x4_t*)(p); }
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
__device__ __forceinline__ f16x4_t zero_h4() { return f16x4_t{0, 0, 0, 0}; }
__device__ __forceinline__ f32x4 mfma32(f16x8_t x, f16x8_t y, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(x, y, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(f16x4_t x, f16x4_t y) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(x, y, zero4(), 0, 0, 0);
}

// Transposing read (gfx950): in each group of 16 lanes, lane 4a + e receives
// element e of the 8-byte units addressed by lanes a, a + 4, a + 8, a + 12 of
// the group.  Used to read K^T fragments straight from the K rows.
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_tr_t;
__device__ __forceinline__ f16x4_t ld4_tr(const hb* p) {
  return __builtin_bit_cast(f16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_tr_t*)(p)));
}

// A fragment of k tiles (q, q + 1) in the register-B order.
__device__ __forceinline__ f16x8_t fragA2(const hb* arow, int q, int g) {
  return cat8(ld4(arow + 16 * q + 4 * g), ld4(arow + 16 * q + 16 + 4 * g));
}
__device__ __forceinline__ f16x8_t tof16x8(f32x4 u, f32x4 v) { return cat8(tof16(u), tof16(v)); }
// The same for the d-contracted K and Q rows at k-step p (columns 32 p ..):
// when D = 16 (mod 32) the last step's upper 16 columns are past the row and
// read as zero (their partner state rows are zero too).
template <int D>
__device__ __forceinline__ f16x8_t fragK(const hb* row, int p, int g) {
  if (32 * p + 16 < D) return fragA2(row, 2 * p, g);
  return cat8(ld4(row + 32 * p + 4 * g), zero_h4());
}
__device__ __forceinline__ f32x4 ld4f(const float* p) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  return f32x4{v.x, v.y, v.z, v.w};
}

// Rows of one sub-chunk [t0, t0 + n) in scan order: scan row i is token
// ta + sgn i.  Element offsets are formed as a wave-uniform part (row base and
// the row's uniform step) plus one small per-lane offset, so that no per-row
// 64-bit offsets stay live across the sub-chunk loop.
struct Sub {
  long long ta;   // token of scan row 0
  long long t0;   // first token of the sub-chunk in original order
  int sgn;        // +1: forward scan, -1: reversed scan
  int r0;         // scan row 0 relative to t0 (so scan row i is t0 + r0 + sgn i)
  int n;          // rows present
};

__device__ __forceinline__ Sub make_sub(long long t0, int n, bool rev) {
  Sub s;
  s.ta = rev ? t0 + n - 1 : t0;
  s.t0 = t0;
  s.sgn = rev ? -1 : 1;
  s.r0 = rev ? n - 1 : 0;
  s.n = n;
  return s;
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
// Note: with this toolchain __builtin_bit_cast of a vector element
// (bit_cast<T>(v[i])) yields element 0 for every i; only whole vectors are
// bit-cast here.

// Raw buffer over the n rows [t0, t0 + n) of a token-major tensor, starting at
// one head's first element.  Offsets past the n rows (and the wrapped
// "negative" offsets of scan rows past n in a reversed scan) are outside the
// buffer: loads there return 0 and stores are dropped by the hardware range
// check, so a ragged sub-chunk needs no branches (a branch around a load would
// make the compiler wait for every outstanding load at the merge).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, long long bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// exp2 of a non-positive argument (results below 2^-126 flush to zero).
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Raw buffer access to a small fp32 block (a state): one per-lane byte offset
// plus a wave-uniform one, so that a state's 4 MD addresses per lane are not
// materialised as separate 64-bit pointers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const float* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ float block_load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
__device__ __forceinline__ void block_store(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, float x) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), r, voff, soff, 0);
}

// Segment start states and the Q half of the segment maps are kept transposed
// in the workspace (element [i][j] at [j][i]): an accumulator tile's four
// values per lane (rows 4g .. 4g+3 of one column) are then four consecutive
// floats, one 128-bit access instead of four.
__device__ __forceinline__ f32x4 tile_load_t(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ void tile_store_t(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, f32x4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, x), r, voff, soff, 0);
}

// --- staging --------------------------------------------------------------------
// Strip-wave thread j holds scan rows 2 (j / (D/8)) and 2 (j / (D/8)) + 1,
// components 8 (j % (D/8)) .. + 7, of K, V and (output pass) Q, so that a
// wavefront's loads cover whole rows; the helper wave holds
// one token's log-gate and beta per lane.  Loading into registers is split from
// writing LDS so that the loads of sub-chunk c+2 are in flight while sub-chunk
// c is computed.  Every load is unconditional: rows past n (and sub-chunks past
// the segment, given as n = 0) read as zeros through the buffer range check.
// Feature prologue factors of (b, h): pairs (fk, fq) of tokens t0 - 1 .. t0 + 64
// of the padded per-head array (a pad pair of zeros before token 0 and after
// token T - 1), so that the pair of rows (t, t + 1), t >= t0 - 1, is one
// 16-byte load at byte (t - t0 + 1) * 8.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t fac_rsrc(const Args& a, int b, int h, long long t0) {
  const long long i0 = ((long long)b * a.H + h) * (a.T + 2) + t0;   // pair of token t0 - 1
  const long long avail = a.T - t0 + 2;                             // pairs through the trailing pad
  return rows_rsrc(a.fac + 2 * i0, (avail < CH + 2 ? avail : CH + 2) * 8);
}

struct StageKQ {
  uint4 k[2], q[2];
  float fk[2], fq[2];   // feature prologue factors of the two rows
};
struct StageV {
  uint4 v[2];
};
struct StageG {
  float g, b;
};

template <int D, bool OUT, bool PRO>
__device__ __forceinline__ void fetch_kq(const Args& a, int b, int h, const Sub& sb, StageKQ& st) {
  const int t = threadIdx.x, i2 = t / (D / 8), c8 = t % (D / 8);
  const int HD = a.H * D;
  const long long e0 = ((long long)b * a.T + sb.t0) * HD + (long long)h * D;
  const __amdgpu_buffer_rsrc_t rk = rows_rsrc(a.k + e0, (long long)sb.n * HD * 2);
  const __amdgpu_buffer_rsrc_t rq = rows_rsrc(a.q + e0, OUT ? (long long)sb.n * HD * 2 : 0);
  const int lr = sb.r0 + sb.sgn * 2 * i2;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const uint32_t off = (uint32_t)((lr + sb.sgn * r) * HD * 2 + 16 * c8);
    const u32x4_t vk = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
    st.k[r] = make_uint4(vk[0], vk[1], vk[2], vk[3]);
    if constexpr (OUT) {
      const u32x4_t vq = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
      st.q[r] = make_uint4(vq[0], vq[1], vq[2], vq[3]);
    }
  }
  if constexpr (PRO) {
    // rows lr and lr + sgn are adjacent tokens: one load of their two pairs
    // (lower token first); rows past the sub-chunk read real neighbours or
    // zeros, and their K/Q rows are zero anyway
    const int lo = sb.sgn > 0 ? lr : lr - 1;   // sub-chunk row of the lower token
    const __amdgpu_buffer_rsrc_t rf = fac_rsrc(a, b, h, sb.t0);
    if constexpr (OUT) {
      const f32x4 f = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rf, (uint32_t)((lo + 1) * 8), 0, 0));
      const bool up = sb.sgn > 0;
      st.fk[0] = up ? f[0] : f[2];
      st.fq[0] = up ? f[1] : f[3];
      st.fk[1] = up ? f[2] : f[0];
      st.fq[1] = up ? f[3] : f[1];
    } else {
      // the map kernels need the key factors only (and have few registers)
#pragma unroll
      for (int r = 0; r < 2; ++r)
        st.fk[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                 rf, (uint32_t)((lr + sb.sgn * r + 1) * 8), 0, 0));
    }
  }
}

__device__ __forceinline__ void fetch_gates(const Args& a, int b, int h, const Sub& sb, StageG& st) {
  const int i = threadIdx.x & 63;
  const long long go = ((long long)b * a.T + sb.t0) * a.H + h;
  const uint32_t off = (uint32_t)((sb.r0 + sb.sgn * i) * a.H * 4);
  st.g = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rows_rsrc(a.g + go, (long long)sb.n * a.H * 4), off, 0, 0));
  st.b = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rows_rsrc(a.beta + go, (long long)sb.n * a.H * 4), off, 0, 0));
}

// V rows in the same thread mapping.
template <int D>
__device__ __forceinline__ void fetch_v(const Args& a, int b, int h, const Sub& sb, StageV& st) {
  const int t = threadIdx.x, i2 = t / (D / 8), c8 = t % (D / 8);
  const int HD = a.H * D;
  const long long e0 = ((long long)b * a.T + sb.t0) * HD + (long long)h * D;
  const __amdgpu_buffer_rsrc_t rv = rows_rsrc(a.v + e0, (long long)sb.n * HD * 2);
  const int lr = sb.r0 + sb.sgn * 2 * i2;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const uint32_t off = (uint32_t)((lr + sb.sgn * r) * HD * 2 + 16 * c8);
    const u32x4_t vv = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
    st.v[r] = make_uint4(vv[0], vv[1], vv[2], vv[3]);
  }
}
template <int D>
__device__ __forceinline__ void stage_v(const Buf& B, const StageV& st) {
  const int t = threadIdx.x, i2 = t / (D / 8), c8 = t % (D / 8);
#pragma unroll
  for (int r = 0; r < 2; ++r) *reinterpret_cast<uint4*>(B.vr + (2 * i2 + r) * Geo<D>::LDV + 8 * c8) = st.v[r];
}

// Write the staged rows into buffer B: K and Q as fp16 (PRO: the key
// features ReLU(f_k k) and the normalised queries f_q q).
template <int D, bool OUT, bool PRO>
__device__ __forceinline__ void stage_kq(const Buf& B, const StageKQ& st) {
  const int t = threadIdx.x, i2 = t / (D / 8), c8 = t % (D / 8);
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    *reinterpret_cast<uint4*>(B.kr + krow<D>(2 * i2 + r) + 8 * c8) =
        PRO ? bf16x8_scaled_f16x8<true>(st.k[r], st.fk[r]) : bf16x8_to_f16x8(st.k[r]);
    if constexpr (OUT)
      *reinterpret_cast<uint4*>(B.qr + krow<D>(2 * i2 + r) + 8 * c8) =
          PRO ? bf16x8_scaled_f16x8<false>(st.q[r], st.fq[r]) : bf16x8_to_f16x8(st.q[r]);
  }
}

// Inclusive prefix sum over the 64 lanes of a wavefront with DPP moves: a
// Hillis-Steele scan inside each row of 16 lanes (shifts 1, 2, 4, 8), then
// row 0's total into row 1, row 2's into row 3 (broadcast of lane 15 / 47),
// and the sum of rows 0-1 into rows 2-3 (broadcast of lane 31).
__device__ __forceinline__ float wave_prefix_sum(float x) {
  int v = __builtin_bit_cast(int, x);
#define GDN_DPP_ADD(ctrl, rmask, bz)                                                                   \
  v = __builtin_bit_cast(int, __builtin_bit_cast(float, v) +                                          \
                                  __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, ctrl, rmask, 0xf, bz)))
  GDN_DPP_ADD(0x111, 0xf, true);    // row_shr:1 (lanes without a source read 0)
  GDN_DPP_ADD(0x112, 0xf, true);    // row_shr:2
  GDN_DPP_ADD(0x114, 0xf, true);    // row_shr:4
  GDN_DPP_ADD(0x118, 0xf, true);    // row_shr:8
  GDN_DPP_ADD(0x142, 0xa, false);   // row_bcast:15 into rows 1 and 3 (other rows add 0)
  GDN_DPP_ADD(0x143, 0xc, false);   // row_bcast:31 into rows 2 and 3
#undef GDN_DPP_ADD
  return __builtin_bit_cast(float, v);
}

// The scan-order gate cumsum in log2 units and the per-token factors (helper).
__device__ __forceinline__ void stage_gates(const Buf& B, const StageG& st, float c) {
  const int i = threadIdx.x & 63;
  const float s = wave_prefix_sum(st.g * kLog2e);
  const float last = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), 63));
  const float e = ex2(s);
  B.g2[i] = s;
  B.eg[i] = e;
  B.ce[i] = c * e;
  B.dn[i] = c * ex2(last - s);
  B.bt[i] = st.b;
}

__device__ void tinv_diag(const Inv& I, const Buf& B);

// Software-pipelined products.  The fragments of a product are read PD steps
// ahead of the MFMAs that use them, and a scheduling fence after every step
// keeps that order (left to itself the compiler places each read one or two
// MFMAs before its use, so every MFMA waits out most of an LDS round trip).
// PD fragments of two reads each stay within the 15 LDS operations a
// wavefront can have in flight.  Measured on the 60 s clip: output launches
// 0.67 -> 0.61 ms (the kernels are bound by their instruction issue: two
// wavefronts per SIMD keep it busy about 80% of the time).
constexpr int kPD = 6;
#define GDN_FENCE() __builtin_amdgcn_sched_barrier(0)

// acc[j][mt] = rows (16 mt ..) of `rows` (d-contracted fp16) times strip j
// (TR: the transposed product, strip as the A operand).
template <int D, int SPW, bool TR, int PD = kPD>
__device__ __forceinline__ void wrows_state(const hb* rows, const f16x8_t (&Xp)[SPW][Geo<D>::NP], int cl, int g,
                                            f32x4 (&acc)[SPW][4]) {
  constexpr int NP = Geo<D>::NP, NF = NP * 4;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int j = 0; j < SPW; ++j) acc[j][mt] = zero4();
  f16x8_t fr[NF];
  auto ld = [&](int i) { fr[i] = fragK<D>(rows + krow<D>(16 * (i & 3) + cl), i >> 2, g); };
#pragma unroll
  for (int i = 0; i < PD && i < NF; ++i) ld(i);
#pragma unroll
  for (int i = 0; i < NF; ++i) {
    GDN_FENCE();
    const int mt = i & 3, p = i >> 2;
#pragma unroll
    for (int j = 0; j < SPW; ++j)
      acc[j][mt] = TR ? mfma32(Xp[j][p], fr[i], acc[j][mt]) : mfma32(fr[i], Xp[j][p], acc[j][mt]);
    if (i + PD < NF) ld(i + PD);
  }
  GDN_FENCE();
}

// out[j][mt] (+)= lower-triangular token matrix M times the token-row tiles
// of strip j (pairs vp[j][0] = (0, 1), vp[j][1] = (2, 3)); TR: transposed.
template <int SPW, bool TR>
__device__ __forceinline__ void wtri(const hb* M, const f16x8_t (&vp)[SPW][2], int cl, int g, f32x4 (&acc)[SPW][4]) {
  constexpr int kP[6] = {0, 0, 0, 0, 1, 1}, kM[6] = {0, 1, 2, 3, 2, 3};
  f16x8_t fr[6];
#pragma unroll
  for (int i = 0; i < 6; ++i) fr[i] = fragA2(M + (16 * kM[i] + cl) * LDT, 2 * kP[i], g);
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    GDN_FENCE();
#pragma unroll
    for (int j = 0; j < SPW; ++j)
      acc[j][kM[i]] = TR ? mfma32(vp[j][kP[i]], fr[i], acc[j][kM[i]]) : mfma32(fr[i], vp[j][kP[i]], acc[j][kM[i]]);
  }
  GDN_FENCE();
}

// X[j] <- dec X[j] + K^T vs[j] (see state_update): K^T fragments by
// transposing reads, pipelined like the products above.
template <int D, int SPW, int PD = kPD>
__device__ __forceinline__ void wstate_update(const hb* kr, const f16x8_t (&vs)[SPW][2], float dec, int cl, int g,
                                              f32x4 (&X)[SPW][Geo<D>::MD]) {
  constexpr int MD = Geo<D>::MD, NF = 2 * MD;
  const hb* kt = kr + krow<D>(4 * g + (cl >> 2)) + 4 * (cl & 3);
  f16x8_t fr[NF];
  // fragment i: token half q = i / MD, component tile md = i % MD
  auto ld = [&](int i) {
    const int q = i / MD, md = i % MD;
    fr[i] = cat8(ld4_tr(kt + krow<D>(32 * q) + 16 * md), ld4_tr(kt + krow<D>(32 * q + 16) + 16 * md));
  };
#pragma unroll
  for (int i = 0; i < PD && i < NF; ++i) ld(i);
#pragma unroll
  for (int md = 0; md < MD; ++md)
#pragma unroll
    for (int j = 0; j < SPW; ++j) X[j][md] = X[j][md] * dec;
#pragma unroll
  for (int i = 0; i < NF; ++i) {
    GDN_FENCE();
    const int q = i / MD, md = i % MD;
#pragma unroll
    for (int j = 0; j < SPW; ++j) X[j][md] = mfma32(fr[i], vs[j][q], X[j][md]);
    if (i + PD < NF) ld(i + PD);
  }
  GDN_FENCE();
}

// NK Gram tiles (see gram_tile), every k step's two fragments read PDG steps
// ahead of its MFMA; consecutive MFMAs update different tiles.
template <int D, int NK, int PDG = 3>
__device__ __forceinline__ void gram_tiles_pl(const hb* const (&ar)[NK], const hb* const (&br)[NK], int g,
                                              f32x4 (&acc)[NK]) {
  constexpr int NP = Geo<D>::NP, NS = NP * NK;
#pragma unroll
  for (int k = 0; k < NK; ++k) acc[k] = zero4();
  f16x8_t fa[NS], fb[NS];
  // step i: k step i / NK of tile i % NK
  auto ld = [&](int i) {
    fa[i] = fragK<D>(ar[i % NK], i / NK, g);
    fb[i] = fragK<D>(br[i % NK], i / NK, g);
  };
#pragma unroll
  for (int i = 0; i < PDG && i < NS; ++i) ld(i);
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    GDN_FENCE();
    acc[i % NK] = mfma32(fa[i], fb[i], acc[i % NK]);
    if (i + PDG < NS) ld(i + PDG);
  }
  GDN_FENCE();
}

// --- Gram tiles -------------------------------------------------------------------
// Tile (ta, tb), ta <= tb, of the products of the K rows of block ta with the
// K (or Q) rows of block tb: lane holds rows y = 16 ta + 4g + r against row
// x = 16 tb + (lane % 16), i.e. entries [x][y .. y+3] of A or P.
template <int D>
__device__ __forceinline__ f32x4 gram_tile(const hb* kr, const hb* xr, int ta, int tb, int cl, int g) {
  using G = Geo<D>;
  const hb* arow = kr + krow<D>(16 * ta + cl);
  const hb* brow = xr + krow<D>(16 * tb + cl);
  f32x4 acc = zero4();
  // both operands in the same (permuted) k order, two 8-byte reads each
#pragma unroll
  for (int p = 0; p < G::NP; ++p) acc = mfma32(fragK<D>(arow, p, g), fragK<D>(brow, p, g), acc);
  return acc;
}

// Lower-triangular 16x16-tile pairs (a <= b) of a 4x4 tile grid, 2 bits per
// pair index (in registers, no table load); the first six are the strictly
// lower ones: (0,1) (0,2) (0,3) (1,2) (1,3) (2,3) (0,0) (1,1) (2,2) (3,3).
constexpr uint32_t pack_pairs(const int (&v)[10]) {
  uint32_t r = 0;
  for (int i = 0; i < 10; ++i) r |= (uint32_t)v[i] << (2 * i);
  return r;
}
constexpr int kPairA[10] = {0, 0, 0, 1, 1, 2, 0, 1, 2, 3};
constexpr int kPairB[10] = {1, 2, 3, 2, 3, 3, 0, 1, 2, 3};
constexpr uint32_t kPackA = pack_pairs(kPairA), kPackB = pack_pairs(kPairB);

// Helper: the diagonal 16x16 blocks of A of sub-chunk B (fp32), then their
// inverses.  The four products are formed before any result is stored: a
// load placed after an LDS store waits for it (the compiler cannot prove the
// two apart), which would serialise the blocks.
template <int D, int PDG = 3>
__device__ void gram_stage_helper(const Args& a, const Buf& B, const Inv& I) {
  const int lane = threadIdx.x & 63, g = lane >> 4, cl = lane & 15;
  const float c2 = a.c * a.c;
  {
    f32x4 sb[4];
    if constexpr (PDG == 0) {
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) sb[blk] = gram_tile<D>(B.kr, B.kr, blk, blk, cl, g);
    } else {
      const hb* const rows[4] = {B.kr + krow<D>(cl), B.kr + krow<D>(16 + cl), B.kr + krow<D>(32 + cl),
                                 B.kr + krow<D>(48 + cl)};
      gram_tiles_pl<D, 4, PDG>(rows, rows, g, sb);
    }
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      const f32x4 s = sb[blk];
      const int x = 16 * blk + cl, y0 = 16 * blk + 4 * g;
      const float gx = B.g2[x], bx = c2 * B.bt[x];
      const f32x4 gy = ld4f(B.g2 + y0);
      float4 v;
      v.x = (x > y0 + 0) ? bx * s[0] * ex2(gx - gy[0]) : 0.f;
      v.y = (x > y0 + 1) ? bx * s[1] * ex2(gx - gy[1]) : 0.f;
      v.z = (x > y0 + 2) ? bx * s[2] * ex2(gx - gy[2]) : 0.f;
      v.w = (x > y0 + 3) ? bx * s[3] * ex2(gx - gy[3]) : 0.f;
      *reinterpret_cast<float4*>(I.ad + blk * ADB + cl * 16 + 4 * g) = v;
    }
    wave_lds_sync();
    tinv_diag(I, B);
  }
}

// Strip waves: the off-diagonal blocks of A (fp16) and, for the output pass,
// P = c tril(Q K^T) * E.  Wave w takes tiles w, w + NSW, ...; the products of
// all its tiles are formed before any epilogue, so that their LDS reads and
// MFMAs overlap (the first NFULL tiles of every wave need no branch), and the
// epilogues read their gate factors before their first store.  The output
// kernel forms the products before it stages its outputs and runs the
// epilogues after (a read placed after an LDS store waits for it).
template <int D, bool OUT>
struct GramStrips {
  static constexpr int NTILE = OUT ? 16 : 6;
  static constexpr int NK = (NTILE + Geo<D>::NSW - 1) / Geo<D>::NSW, NFULL = NTILE / Geo<D>::NSW;
};
template <int D, bool OUT, int PDG = 3>
__device__ __forceinline__ void gram_strips_products(const Buf& B, f32x4 (&sk)[GramStrips<D, OUT>::NK]) {
  using GS = GramStrips<D, OUT>;
  const int wave = wave_id(), lane = threadIdx.x & 63, g = lane >> 4, cl = lane & 15;
  if constexpr (PDG == 0) {   // each tile's fragments read just before its MFMAs
#pragma unroll
    for (int k = 0; k < GS::NK; ++k) {
      const int t = wave + k * Geo<D>::NSW;
      if (k < GS::NFULL || t < GS::NTILE) {
        const bool isp = t >= 6;
        const int u = isp ? t - 6 : t;
        const int ta = (kPackA >> (2 * u)) & 3, tb = (kPackB >> (2 * u)) & 3;
        sk[k] = gram_tile<D>(B.kr, isp ? B.qr : B.kr, ta, tb, cl, g);
      }
    }
    return;
  }
  auto rows = [&](int k, const hb*& ar, const hb*& br) {
    const int t = wave + k * Geo<D>::NSW;
    const bool isp = t >= 6;
    const int u = isp ? t - 6 : t;
    const int ta = (kPackA >> (2 * u)) & 3, tb = (kPackB >> (2 * u)) & 3;
    ar = B.kr + krow<D>(16 * ta + cl);
    br = (isp ? B.qr : B.kr) + krow<D>(16 * tb + cl);
  };
  if constexpr (GS::NFULL > 0) {
    const hb* ar[GS::NFULL];
    const hb* br[GS::NFULL];
#pragma unroll
    for (int k = 0; k < GS::NFULL; ++k) rows(k, ar[k], br[k]);
    f32x4 acc[GS::NFULL];
    gram_tiles_pl<D, GS::NFULL, PDG>(ar, br, g, acc);
#pragma unroll
    for (int k = 0; k < GS::NFULL; ++k) sk[k] = acc[k];
  }
  if constexpr (GS::NK > GS::NFULL) {
    if (wave + GS::NFULL * Geo<D>::NSW < GS::NTILE) {   // wave-uniform
      const hb* ar[1];
      const hb* br[1];
      rows(GS::NFULL, ar[0], br[0]);
      f32x4 acc[1];
      gram_tiles_pl<D, 1, PDG>(ar, br, g, acc);
      sk[GS::NFULL] = acc[0];
    }
  }
}
template <int D, bool OUT>
__device__ __forceinline__ void gram_strips_epilogues(const Args& a, const Buf& B, const Inv& I,
                                                      const f32x4 (&sk)[GramStrips<D, OUT>::NK]) {
  using GS = GramStrips<D, OUT>;
  const int wave = wave_id(), lane = threadIdx.x & 63, g = lane >> 4, cl = lane & 15;
  const float c2 = a.c * a.c;
  float gx[GS::NK], bx[GS::NK];
  f32x4 gy[GS::NK];
#pragma unroll
  for (int k = 0; k < GS::NK; ++k) {
    const int t = wave + k * Geo<D>::NSW;
    if (!(k < GS::NFULL || t < GS::NTILE)) continue;
    const bool isp = t >= 6;
    const int u = isp ? t - 6 : t;
    const int ta = (kPackA >> (2 * u)) & 3, tb = (kPackB >> (2 * u)) & 3;
    const int x = 16 * tb + cl, y0 = 16 * ta + 4 * g;
    gx[k] = B.g2[x];
    gy[k] = ld4f(B.g2 + y0);
    bx[k] = isp ? a.c : c2 * B.bt[x];
  }
#pragma unroll
  for (int k = 0; k < GS::NK; ++k) {
    const int t = wave + k * Geo<D>::NSW;
    if (!(k < GS::NFULL || t < GS::NTILE)) continue;
    const bool isp = t >= 6;
    const int u = isp ? t - 6 : t;
    const int ta = (kPackA >> (2 * u)) & 3, tb = (kPackB >> (2 * u)) & 3;
    const f32x4 s = sk[k];
    const int x = 16 * tb + cl, y0 = 16 * ta + 4 * g;
    const float f = bx[k], gxx = gx[k];
    const f32x4 gyy = gy[k];
    if (!isp) {
      store4_h(I.ao + x * LDT + y0, f * s[0] * ex2(gxx - gyy[0]), f * s[1] * ex2(gxx - gyy[1]),
               f * s[2] * ex2(gxx - gyy[2]), f * s[3] * ex2(gxx - gyy[3]));
    } else {
      store4_h(B.pp + x * LDT + y0, (x >= y0 + 0) ? f * s[0] * ex2(gxx - gyy[0]) : 0.f,
               (x >= y0 + 1) ? f * s[1] * ex2(gxx - gyy[1]) : 0.f, (x >= y0 + 2) ? f * s[2] * ex2(gxx - gyy[2]) : 0.f,
               (x >= y0 + 3) ? f * s[3] * ex2(gxx - gyy[3]) : 0.f);
    }
  }
}
template <int D, bool OUT, int PDG = 3>
__device__ void gram_stage_strips(const Args& a, const Buf& B, const Inv& I) {
  f32x4 sk[GramStrips<D, OUT>::NK];
  gram_strips_products<D, OUT, PDG>(B, sk);
  gram_strips_epilogues<D, OUT>(a, B, I, sk);
}

// --- triangular inverse (helper wavefront) ------------------------------------------
// Tm = (I + A)^-1 of sub-chunk B into B.tt as Tm diag(beta) (fp16 rows), in
// two parts run in different phases:
// tinv_diag: diagonal 16x16 blocks; lane (block g, row i) solves row i of
//   T_gg (I + A_gg) = I from the last column to the first, in fp32.
// tinv_offdiag: off-diagonal blocks, level by level,
//   T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj,
//   with every T_kj kept in registers in accumulator layout (fp16), so the
//   levels need no LDS round trip.
__device__ void tinv_diag(const Inv& I, const Buf& B) {
  const int lane = threadIdx.x & 63, g = lane >> 4, cl = lane & 15;
  const float* Ab = I.ad + g * ADB;
  float s[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) s[j] = (j == cl) ? 1.f : 0.f;
#pragma unroll
  for (int k = 15; k >= 1; --k) {
    const float tk = s[k];
#pragma unroll
    for (int q = 0; 4 * q < k; ++q) {
      const f32x4 a4 = ld4f(Ab + k * 16 + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * q + e < k) s[4 * q + e] = fmaf(-tk, a4[e], s[4 * q + e]);
    }
  }
  hb* tdr = I.td + (16 * g + cl) * LDD;
  hb* ttr = B.tt + (16 * g + cl) * LDT + 16 * g;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4 bb = ld4f(B.bt + 16 * g + 4 * q);
    store4_h(tdr + 4 * q, s[4 * q], s[4 * q + 1], s[4 * q + 2], s[4 * q + 3]);
    store4_h(ttr + 4 * q, s[4 * q] * bb[0], s[4 * q + 1] * bb[1], s[4 * q + 2] * bb[2], s[4 * q + 3] * bb[3]);
  }
}

// One off-diagonal block T_ij = -T_ii M, M = sum_k A_ik T_kj (the A row
// fragments a0, a1 against the T column pairs p0, p1): returns -T_ij in
// accumulator layout (fp16, for the next level) and (T_ii M)^T in tr (lane
// holds [cl][4g + r]) for the store.
__device__ __forceinline__ f16x4_t tinv_block(f16x8_t a0, f16x8_t p0, bool two, f16x8_t a1, f16x8_t p1,
                                              f16x4_t tii, f32x4& tr) {
  f32x4 m = mfma32(a0, p0, zero4());
  if (two) m = mfma32(a1, p1, m);
  const f16x4_t mh = tof16(m);
  const f32x4 tc = mfma16(tii, mh);          // T_ii M: lane holds [4g + r][cl]
  tr = mfma16(mh, tii);                      // (T_ii M)^T: lane holds [cl][4g + r]
  return tof16(-tc);
}

// Every LDS operand is read first and every result stored last, so that no
// read waits behind a store (see gram_stage_helper).
__device__ void tinv_offdiag(const Inv& I, const Buf& B) {
  const int lane = threadIdx.x & 63, g = lane >> 4, cl = lane & 15;
  // diagonal blocks 0..2 in accumulator layout (lane: rows 4g + r, column cl)
  f16x4_t d[3], tii[3];
  f32x4 bb[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
#pragma unroll
    for (int r = 0; r < 4; ++r) d[j][r] = __builtin_bit_cast(_Float16, I.td[(16 * j + 4 * g + r) * LDD + cl]);
    tii[j] = ld4(I.td + (16 * (j + 1) + cl) * LDD + 4 * g);   // T_{j+1, j+1}, row-operand layout
    bb[j] = ld4f(B.bt + 16 * j + 4 * g);
  }
  auto arow = [&](int i, int j) { return I.ao + (16 * i + cl) * LDT + 16 * j; };
  const f16x8_t a10 = fragA2(arow(1, 0), 0, g), a21 = fragA2(arow(2, 1), 0, g), a32 = fragA2(arow(3, 2), 0, g);
  const f16x8_t a20 = fragA2(arow(2, 0), 0, g), a31 = fragA2(arow(3, 1), 0, g);
  const f16x8_t a30 = fragA2(arow(3, 0), 0, g), a30b = fragA2(arow(3, 0), 2, g);
  const f16x4_t z = zero_h4();
  const f16x8_t zz = cat8(z, z);
  f32x4 tr[6];
  const f16x4_t t10 = tinv_block(a10, cat8(d[0], z), false, zz, zz, tii[0], tr[0]);
  const f16x4_t t21 = tinv_block(a21, cat8(d[1], z), false, zz, zz, tii[1], tr[1]);
  (void)tinv_block(a32, cat8(d[2], z), false, zz, zz, tii[2], tr[2]);
  const f16x4_t t20 = tinv_block(a20, cat8(d[0], t10), false, zz, zz, tii[1], tr[3]);
  (void)tinv_block(a31, cat8(d[1], t21), false, zz, zz, tii[2], tr[4]);
  (void)tinv_block(a30, cat8(d[0], t10), true, a30b, cat8(t20, z), tii[2], tr[5]);
  // Tm diag(beta) blocks (i, j): rows 16 i + cl, columns 16 j + 4g ..
  constexpr int bi[6] = {1, 2, 3, 2, 3, 3}, bj[6] = {0, 1, 2, 0, 1, 0};
#pragma unroll
  for (int k = 0; k < 6; ++k)
    store4_h(B.tt + (16 * bi[k] + cl) * LDT + 16 * bj[k] + 4 * g, -tr[k][0] * bb[bj[k]][0],
             -tr[k][1] * bb[bj[k]][1], -tr[k][2] * bb[bj[k]][2], -tr[k][3] * bb[bj[k]][3]);
}

// --- reuse of the inverse ----------------------------------------------------------
// The map kernels store every sub-chunk's Tm diag(beta) and the output kernels
// of the same scan load it instead of forming and inverting I + A again: the
// same sub-chunks, rows and arithmetic, so the blocks are bit-identical.  Per
// sub-chunk the 10 lower 16x16 blocks (the upper ones are zero) as 320 pieces
// of 16 bytes: piece k is half k % 2 of row (k / 2) % 16 of block k / 32, the
// blocks in the order (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) .. (3,3).
constexpr int kTmPieces = 320;
constexpr int kTmElems = kTmPieces * 8;   // fp16 elements per sub-chunk
constexpr int kTmRowBlk[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
constexpr int kTmColBlk[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};
constexpr uint32_t kPackTr = pack_pairs(kTmRowBlk), kPackTc = pack_pairs(kTmColBlk);

// Element offset of piece k in a Tm rows buffer (B.tt).
__device__ __forceinline__ int tm_piece_lds(int k) {
  const int blk = k >> 5, r = (k >> 1) & 15, half = k & 1;
  const int bi = (kPackTr >> (2 * blk)) & 3, bj = (kPackTc >> (2 * blk)) & 3;
  return (16 * bi + r) * LDT + 16 * bj + 8 * half;
}

// The Tm blocks of sub-chunk sb of scan slot `slot` (empty for n = 0, or
// without a Tm buffer).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tm_rsrc(const Args& a, int slot, int b, int h, const Sub& sb) {
  const long long U = (a.T + CH - 1) / CH;
  const hb* p = a.tm + ((((long long)slot * a.B + b) * a.H + h) * U + sb.t0 / CH) * kTmElems;
  return rows_rsrc(p, a.tm != nullptr && sb.n > 0 ? kTmElems * 2 : 0);
}

// Map kernels (strip waves): store the Tm blocks of buffer B.  Every lane
// issues the same stores; pieces past 320 read a valid LDS address and fall
// outside the buffer.
template <int D>
__device__ __forceinline__ void store_tm(__amdgpu_buffer_rsrc_t r, const Buf& B) {
  constexpr int NTS = 64 * Geo<D>::NSW, NI = (kTmPieces + NTS - 1) / NTS;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int k = (int)threadIdx.x + NTS * i;
    const uint4 x = *reinterpret_cast<const uint4*>(B.tt + tm_piece_lds(k < kTmPieces ? k : kTmPieces - 1));
    __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{x.x, x.y, x.z, x.w}, r, (uint32_t)(16 * k), 0, 0);
  }
}

// Output kernels (helper wave): five pieces per lane.
struct StageTm {
  uint4 x[5];
};
__device__ __forceinline__ void fetch_tm(__amdgpu_buffer_rsrc_t r, StageTm& st) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)(16 * (lane + 64 * i)), 0, 0);
    st.x[i] = make_uint4(v[0], v[1], v[2], v[3]);
  }
}
__device__ __forceinline__ void stage_tm(const Buf& B, const StageTm& st) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 5; ++i) *reinterpret_cast<uint4*>(B.tt + tm_piece_lds(lane + 64 * i)) = st.x[i];
}

// P tiles t0, t0 + dt, .. (below 10) of sub-chunk B: P = c tril(Q K^T) * E,
// products first, then epilogues (gate factors read before the first store).
template <int D, int NK>
__device__ __forceinline__ void gram_p_products(const Buf& B, int t0, int dt, f32x4 (&sk)[NK]) {
  const int lane = threadIdx.x & 63, g = lane >> 4, cl = lane & 15;
  // every caller's tiles are all below 10 or (a single tile) none is (wave-uniform)
  if (t0 + (NK - 1) * dt >= 10) return;
  const hb* ar[NK];
  const hb* br[NK];
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    const int u = t0 + k * dt;
    const int ta = (kPackA >> (2 * u)) & 3, tb = (kPackB >> (2 * u)) & 3;
    ar[k] = B.kr + krow<D>(16 * ta + cl);
    br[k] = B.qr + krow<D>(16 * tb + cl);
  }
  gram_tiles_pl<D, NK>(ar, br, g, sk);
}
template <int NK>
__device__ __forceinline__ void gram_p_epilogues(const Args& a, const Buf& B, int t0, int dt, const f32x4 (&sk)[NK]) {
  const int lane = threadIdx.x & 63, g = lane >> 4, cl = lane & 15;
  float gx[NK];
  f32x4 gy[NK];
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    const int u = t0 + k * dt;
    if (u >= 10) continue;
    const int ta = (kPackA >> (2 * u)) & 3, tb = (kPackB >> (2 * u)) & 3;
    gx[k] = B.g2[16 * tb + cl];
    gy[k] = ld4f(B.g2 + 16 * ta + 4 * g);
  }
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    const int u = t0 + k * dt;
    if (u >= 10) continue;
    const int ta = (kPackA >> (2 * u)) & 3, tb = (kPackB >> (2 * u)) & 3;
    const f32x4 s = sk[k];
    const int x = 16 * tb + cl, y0 = 16 * ta + 4 * g;
    const float gxx = gx[k], cc = a.c;
    const f32x4 gyy = gy[k];
    store4_h(B.pp + x * LDT + y0, (x >= y0 + 0) ? cc * s[0] * ex2(gxx - gyy[0]) : 0.f,
             (x >= y0 + 1) ? cc * s[1] * ex2(gxx - gyy[1]) : 0.f, (x >= y0 + 2) ? cc * s[2] * ex2(gxx - gyy[2]) : 0.f,
             (x >= y0 + 3) ? cc * s[3] * ex2(gxx - gyy[3]) : 0.f);
  }
}
template <int D, int NK>
__device__ __forceinline__ void gram_p_tiles(const Args& a, const Buf& B, int t0, int dt) {
  f32x4 sk[NK];
  gram_p_products<D, NK>(B, t0, dt, sk);
  gram_p_epilogues<NK>(a, B, t0, dt, sk);
}
// With the inverse loaded, the helper forms the last kHelperP(NSW) P tiles and
// the strip waves one each of the rest.
constexpr int kHelperP(int nsw) { return 10 - nsw > 3 ? 10 - nsw : 3; }

// --- strip-wave products ----------------------------------------------------------
// State strip: X[md] (md = 0 .. MD-1), the 16x16 accumulator tiles of rows
// 16 md .. 16 md + 15 of the wave's 16 state columns, fp32.

// fp16 B pairs of a state strip (tiles 2p, 2p + 1; a missing last tile is 0).
template <int D>
__device__ __forceinline__ void state_pairs(const f32x4 (&X)[Geo<D>::MD], f16x8_t (&Xp)[Geo<D>::NP]) {
  using G = Geo<D>;
#pragma unroll
  for (int p = 0; p < G::NP; ++p)
    Xp[p] = cat8(tof16(X[2 * p]), 2 * p + 1 < G::MD ? tof16(X[2 * p + 1]) : zero_h4());
}

// acc[j][mt] = rows (16 mt ..) of `rows` (d-contracted fp16) times strip j.
template <int D, int SPW>
__device__ __forceinline__ void rows_times_state(const hb* rows, const f16x8_t (&Xp)[SPW][Geo<D>::NP], int cl, int g,
                                                 f32x4 (&acc)[SPW][4]) {
  using G = Geo<D>;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int j = 0; j < SPW; ++j) acc[j][mt] = zero4();
  // k-pair outer, tile inner: consecutive MFMAs update different accumulators
#pragma unroll
  for (int p = 0; p < G::NP; ++p)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const f16x8_t a = fragK<D>(rows + krow<D>(16 * mt + cl), p, g);
#pragma unroll
      for (int j = 0; j < SPW; ++j) acc[j][mt] = mfma32(a, Xp[j][p], acc[j][mt]);
    }
}

// out[j][mt] (+)= lower-triangular token matrix M (fp16 rows, zero above the
// diagonal) times the token-row tiles held as pairs vp[j][0] = (0, 1),
// vp[j][1] = (2, 3).
template <int SPW>
__device__ __forceinline__ void tri_times(const hb* M, const f16x8_t (&vp)[SPW][2], int cl, int g,
                                          f32x4 (&acc)[SPW][4]) {
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int mt = 2 * p; mt < 4; ++mt) {
      const f16x8_t a = fragA2(M + (16 * mt + cl) * LDT, 2 * p, g);
#pragma unroll
      for (int j = 0; j < SPW; ++j) acc[j][mt] = mfma32(a, vp[j][p], acc[j][mt]);
    }
}

// Transposed products for the outputs: out[mt] (+)= (rows x strip)^T, i.e.
// lane (g, cl) receives row 16 mt + cl, strip columns 4g .. 4g + 3 (the state or
// V' tiles are the A operand, the LDS rows the B operand), so that each lane
// stores four consecutive columns of one token.
template <int D>
__device__ __forceinline__ void state_times_rows_T(const hb* rows, const f16x8_t (&Xp)[Geo<D>::NP], int cl, int g,
                                                   f32x4 (&acc)[4]) {
  using G = Geo<D>;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) acc[mt] = zero4();
#pragma unroll
  for (int p = 0; p < G::NP; ++p)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[mt] = mfma32(Xp[p], fragK<D>(rows + krow<D>(16 * mt + cl), p, g), acc[mt]);
}

// X[j] <- dec X[j] + K^T vs[j]  (vs: fp16 pairs of token-row tiles).  The K^T
// fragments are transposing reads of the K rows: lane (g, cl) = (g, a + 4 j)
// addresses row 16 h + 4 g + j, components 16 md + 4 a .. + 3, so that lane
// (g, i) receives component 16 md + i of rows 16 h + 4 g .. + 3, which is the
// register-B token order of vs.
template <int D, int SPW>
__device__ __forceinline__ void state_update(const hb* kr, const f16x8_t (&vs)[SPW][2], float dec, int cl, int g,
                                             f32x4 (&X)[SPW][Geo<D>::MD]) {
  using G = Geo<D>;
#pragma unroll
  for (int md = 0; md < G::MD; ++md)
#pragma unroll
    for (int j = 0; j < SPW; ++j) X[j][md] = X[j][md] * dec;
  const hb* kt = kr + krow<D>(4 * g + (cl >> 2)) + 4 * (cl & 3);
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int md = 0; md < G::MD; ++md) {
      const f16x8_t a = cat8(ld4_tr(kt + krow<D>(32 * q) + 16 * md), ld4_tr(kt + krow<D>(32 * q + 16) + 16 * md));
#pragma unroll
      for (int j = 0; j < SPW; ++j) X[j][md] = mfma32(a, vs[j][q], X[j][md]);
    }
}

// Value tile mt of strip w in accumulator layout (lane (g, cl): rows
// 16 mt + 4 g .. + 3, column 16 w + cl), by one transposing read of the staged
// bf16 V rows: lane (g, a + 4 j) addresses row 16 mt + 4 g + j, columns
// 16 w + 4 a .. + 3.
template <int D>
__device__ __forceinline__ f32x4 vals_tile(const bh* vr, int mt, int w, int cl, int g) {
  const f16x4_t x = ld4_tr(vr + (16 * mt + 4 * g + (cl >> 2)) * Geo<D>::LDV + 16 * w + 4 * (cl & 3));
  const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_shufflevector(x, x, 0, 1));
  const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_shufflevector(x, x, 2, 3));
  return f32x4{__uint_as_float(lo << 16), __uint_as_float(lo & 0xffff0000u), __uint_as_float(hi << 16),
               __uint_as_float(hi & 0xffff0000u)};
}

// ---------------------------------------------------------------------------
// 1. Segment maps.  grid (segments padded to a multiple of 8, B * H).  The state X = [P | Q]
// (D x 2D): strip wave w owns column strip w of P and column strip w of Q.
// QO: Q only (the reversed scan of a bidirectional call, whose P is the
// transpose of the forward scan's: every token's factor a (I - b k k^T) is
// symmetric, so the product in reversed order is the transposed product).
template <int D, bool QO, bool PRO>
__device__ __forceinline__ void seg_map_body(Args a) {
  using G = Geo<D>;
  using L = Lay<D, false>;
  constexpr int MD = G::MD, SPW = QO ? 1 : 2, JQ = SPW - 1;   // JQ: the Q strip
  // Under the Q-only kernels' 128-register cap the products and Gram tiles
  // read each fragment just before its MFMA (the pipelined forms spill there).
  constexpr int PDG = QO ? 0 : 3;
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
  const int wave = wave_id(), lane = threadIdx.x & 63, g = lane >> 4, cl = lane & 15;
  const int pos = blockIdx.x;                       // scan position of the segment
  if (pos >= a.npos) return;                        // padding of the grid (whole workgroup)
  const int bh_ = a.heads_rev ? (int)(gridDim.y - 1 - blockIdx.y) : (int)blockIdx.y, b = bh_ / a.H, h = bh_ % a.H;
  const int slot = a.slot0 + (int)blockIdx.z, dir = dir_of_slot(a.dirs, slot);
  const bool rev = dir == 1;
  const int seg = rev ? a.NS - 1 - pos : pos;
  const long long s0 = (long long)seg * a.L;
  const long long s1 = (s0 + a.L < a.T) ? s0 + a.L : a.T;
  const int nsub = (int)((s1 - s0 + CH - 1) / CH);
  const Inv I = inv_at<D, false>(smem);
  const bool helper = wave == G::HW;

  for (int i = threadIdx.x; i < L::BYTES / 16; i += G::NT) reinterpret_cast<uint4*>(smem)[i] = make_uint4(0, 0, 0, 0);

  f32x4 X[SPW][MD];
#pragma unroll
  for (int md = 0; md < MD; ++md)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (!QO) X[0][md][r] = (wave == md && 4 * g + r == cl) ? 1.f : 0.f;
      X[JQ][md][r] = 0.f;
    }

  auto piece = [&](int jj) {   // sub-chunk jj of the scan; past the segment: empty
    const int jc = rev ? nsub - 1 - jj : jj;
    const long long t0 = jj < nsub ? s0 + (long long)jc * CH : s0;
    return make_sub(t0, jj < nsub ? (int)((s1 - t0) < CH ? (s1 - t0) : CH) : 0, rev);
  };
  StageKQ sk;
  StageV sv;
  StageG sg;
  {
    const Sub s0b = piece(0), s1b = piece(1);
    if (helper) {
      fetch_gates(a, b, h, s0b, sg);
    } else {
      fetch_kq<D, false, PRO>(a, b, h, s0b, sk);
      fetch_v<D>(a, b, h, s0b, sv);
    }
    __syncthreads();
    if (helper) {
      stage_gates(buf_at<D, false>(smem, 0), sg, a.c);
      fetch_gates(a, b, h, s1b, sg);
    } else {
      stage_kq<D, false, PRO>(buf_at<D, false>(smem, 0), sk);
      stage_v<D>(buf_at<D, false>(smem, 0), sv);
      fetch_kq<D, false, PRO>(a, b, h, s1b, sk);
      fetch_v<D>(a, b, h, s1b, sv);
    }
    __syncthreads();
    if (helper) gram_stage_helper<D, PDG>(a, buf_at<D, false>(smem, 0), I);
    else gram_stage_strips<D, false, PDG>(a, buf_at<D, false>(smem, 0), I);
    __syncthreads();
  }
  if (helper) {
    // helper: gate factors of c+1, inverse of c, diagonal A blocks of c+1
    for (int c = 0; c < nsub; ++c) {
      const Buf Bc = buf_at<D, false>(smem, c & 1), Bn = buf_at<D, false>(smem, (c + 1) & 1);
      const Inv I = inv_at<D, false>(smem);
      stage_gates(Bn, sg, a.c);
      fetch_gates(a, b, h, piece(c + 2), sg);
      tinv_offdiag(I, Bc);
      __syncthreads();
      if (c + 1 < nsub) gram_stage_helper<D, PDG>(a, Bn, I);
      __syncthreads();
    }
    return;
  }
  f32x4 R[SPW][4];
  for (int c = 0; c < nsub; ++c) {
    const Buf Bc = buf_at<D, false>(smem, c & 1), Bn = buf_at<D, false>(smem, (c + 1) & 1);
      const Inv I = inv_at<D, false>(smem);
    // alpha
    stage_kq<D, false, PRO>(Bn, sk);
    fetch_kq<D, false, PRO>(a, b, h, piece(c + 2), sk);
    {
      f16x8_t Xp[SPW][G::NP];
#pragma unroll
      for (int j = 0; j < SPW; ++j) state_pairs<D>(X[j], Xp[j]);
      if constexpr (QO) rows_times_state<D, SPW>(Bc.kr, Xp, cl, g, R);
      else wrows_state<D, SPW, false>(Bc.kr, Xp, cl, g, R);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f32x4 ce = ld4f(Bc.ce + 16 * mt + 4 * g);
        if constexpr (!QO) R[0][mt] = -(ce * R[0][mt]);
        R[JQ][mt] = vals_tile<D>(Bc.vr, mt, wave, cl, g) - ce * R[JQ][mt];
      }
    }
    __syncthreads();
    // beta: the V rows of c+1 replace those of c (read in alpha only)
    stage_v<D>(Bc, sv);
    fetch_v<D>(a, b, h, piece(c + 2), sv);
    {
      f16x8_t Rh[SPW][2];
#pragma unroll
      for (int j = 0; j < SPW; ++j) {
        Rh[j][0] = tof16x8(R[j][0], R[j][1]);
        Rh[j][1] = tof16x8(R[j][2], R[j][3]);
      }
      f32x4 Vn[SPW][4];
#pragma unroll
      for (int j = 0; j < SPW; ++j)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) Vn[j][mt] = zero4();
      if constexpr (QO) tri_times<SPW>(Bc.tt, Rh, cl, g, Vn);
      else wtri<SPW, false>(Bc.tt, Rh, cl, g, Vn);
      f16x8_t Vs[SPW][2];
      const f32x4 d0 = ld4f(Bc.dn + 4 * g), d1 = ld4f(Bc.dn + 16 + 4 * g);
      const f32x4 d2 = ld4f(Bc.dn + 32 + 4 * g), d3 = ld4f(Bc.dn + 48 + 4 * g);
#pragma unroll
      for (int j = 0; j < SPW; ++j) {
        Vs[j][0] = tof16x8(Vn[j][0] * d0, Vn[j][1] * d1);
        Vs[j][1] = tof16x8(Vn[j][2] * d2, Vn[j][3] * d3);
      }
      if constexpr (QO) state_update<D, SPW>(Bc.kr, Vs, Bc.eg[CH - 1], cl, g, X);
      else wstate_update<D, SPW>(Bc.kr, Vs, Bc.eg[CH - 1], cl, g, X);
    }
    // The Q-only maps serve bidirectional calls, which never reuse Tm (their
    // a.tm is null: the stores fall outside an empty buffer).  Under the
    // Q-only kernels' 128-register cap the compiler's spill placement depends
    // on this code: with it the plain variant keeps its loop free of spills,
    // without it the prologue variant does (measured at the 60 s clip, per
    // Q-only launch: 0.29 against 0.33 ms, and 0.31 against 0.33 ms).
    if constexpr (!QO || !PRO) store_tm<D>(tm_rsrc(a, slot, b, h, piece(c)), Bc);
    if (c + 1 < nsub) gram_stage_strips<D, false, PDG>(a, Bn, I);
    __syncthreads();
  }
  // store X = [P | Q] ([D][2D], P row-major, Q transposed; QO: the Q half)
  const float* Xg = a.maps + ((((size_t)slot * a.B + b) * a.H + h) * a.NS + pos) * (size_t)D * (2 * D);
  const __amdgpu_buffer_rsrc_t xr = block_rsrc(Xg, D * 2 * D * 4);
  const uint32_t xo = (uint32_t)((4 * g * 2 * D + wave * 16 + cl) * 4);
  if constexpr (!QO) {
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int r = 0; r < 4; ++r) block_store(xr, xo, (uint32_t)((md * 16 + r) * 2 * D * 4), X[0][md][r]);
  }
  const uint32_t xq = (uint32_t)(((wave * 16 + cl) * 2 * D + D + 4 * g) * 4);
#pragma unroll
  for (int md = 0; md < MD; ++md) tile_store_t(xr, xq, (uint32_t)(md * 16 * 4), X[JQ][md]);
}

// [P | Q] maps: one workgroup per CU (LDS and registers).
template <int D, bool PRO>
__global__ __launch_bounds__(Geo<D>::NT) void seg_map_kernel(Args a) {
  seg_map_body<D, false, PRO>(a);
}
// Q-only maps: their LDS allows two workgroups per CU, and asking for four
// wavefronts per SIMD caps the registers at 128 (a few spill at D = 112).
// Measured at the 60 s clip: 0.27 ms against 0.40 ms with one workgroup per CU.
template <int D, bool PRO>
__global__ __launch_bounds__(Geo<D>::NT) __attribute__((amdgpu_waves_per_eu(4))) void seg_map_q_kernel(Args a) {
  seg_map_body<D, true, PRO>(a);
}

// ---------------------------------------------------------------------------
// 2. Segment chain.  grid (B * H, ndir x column groups[, groups]), per head and
// direction one workgroup of MD wavefronts (or two, see ChainSplitCols):
// H_{p+1} = P_p H_p + Q_p over the segments in scan order, i.e. the prefix
// composition of the segments' affine maps.  A wavefront carries the state
// columns of its 16-column strip in fp32 registers.  Each step the
// map P_p is staged once into LDS as split bf16 (x = hi + lo) and the product
// is formed as hi*hi + hi*lo + lo*hi with fp32 accumulation (about 16
// significant bits per operand); the next map is loaded meanwhile.
template <int D>
struct ChainLay {
  static constexpr int MD = D / 16;
  static constexpr int DP = (D + 31) / 32 * 32;
  static constexpr int NP = DP / 32;
  static constexpr int LDC = DP + 8;             // row stride (elements) of a staged map
  static constexpr int MAT = D * LDC * 2;        // one bf16 matrix
  static constexpr int BYTES = 2 * 2 * MAT;      // (hi, lo) x double buffer
  static_assert(BYTES <= 160 * 1024, "workgroup LDS budget exceeded");
};

// CS: the chain of one head and scan runs as NH = 2 workgroups, each with the
// state columns of NW strips (a wavefront per strip, one per SIMD): every
// workgroup stages the whole map P_p, and a wavefront no longer shares its
// SIMD's matrix core with another strip; a strip index past the state (D =
// 112: 7 strips, 2 x 4 wavefronts) computes on zeros and stores nothing.
// Faster per step (the whole chain, latency-bound: 0.40 -> 0.32 ms at the 60 s
// clip; the split chain's chain of group maps, likewise serial) but less work
// per CU, so the split chain's many-workgroup compose and expand launches,
// bound by the GPU's capacity, keep one workgroup of MD wavefronts.
template <int D, bool CS>
struct ChainSplitCols {
  static constexpr int MD = D / 16;
  static constexpr int NH = CS && MD >= 2 ? 2 : 1;
  static constexpr int NW = (MD + NH - 1) / NH;
};

typedef __attribute__((address_space(3))) const volatile s16x4_t lds_s16x4_t;
__device__ __forceinline__ bf16x8_t fragB2(const bh* arow, int q, int g) {
  const s16x4_t x = *(lds_s16x4_t*)(arow + 16 * q + 4 * g);
  const s16x4_t y = *(lds_s16x4_t*)(arow + 16 * q + 16 + 4 * g);
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
}

// fp32 tile -> (hi, lo) bf16 halves, each as 4 raw values: hi = x rounded to
// bf16 (nearest, ties to even), lo = (x - hi) rounded likewise; the
// conversions are packed two values at a time.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split4(f32x4 v, s16x4_t& hi, s16x4_t& lo) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  const uint32_t h01 = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{v[0], v[1]}, bf16x2_t));
  const uint32_t h23 = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{v[2], v[3]}, bf16x2_t));
  const f32x2_t r01{v[0] - __uint_as_float(h01 << 16), v[1] - __uint_as_float(h01 & 0xffff0000u)};
  const f32x2_t r23{v[2] - __uint_as_float(h23 << 16), v[3] - __uint_as_float(h23 & 0xffff0000u)};
  const uint32_t l01 = __builtin_bit_cast(uint32_t, __builtin_convertvector(r01, bf16x2_t));
  const uint32_t l23 = __builtin_bit_cast(uint32_t, __builtin_convertvector(r23, bf16x2_t));
  hi = __builtin_bit_cast(s16x4_t, u32x2_t{h01, h23});
  lo = __builtin_bit_cast(s16x4_t, u32x2_t{l01, l23});
}

// Modes (Args::ch_mode), for chains long enough to be worth splitting:
//   0  the whole chain over positions 0 .. NS-2 from the seed, storing every
//      start state and the final one (position NS-1);
//   1  compose: group g = blockIdx.z / 2 covers positions [g m, g m + m) (the
//      last group fewer); part blockIdx.z % 2 = 0 runs its maps from I
//      without Q (the product P_g), part 1 from 0 with Q (Q_g): the group's
//      affine map, stored in gmaps like a segment map (P row-major, Q^T);
//   2  the chain over the group maps from the seed, storing each group's
//      start state in gstarts;
//   3  expand: group g = blockIdx.z from its start state over its positions,
//      storing every start state (the last group also the final one).
// Serial steps: 2m + G instead of NS-1 (m ~ sqrt((NS-1)/2)), at the cost of
// reading every map twice.
template <int D, bool PT, bool CS>
__global__ __launch_bounds__((64 * ChainSplitCols<D, CS>::NW)) void seg_chain_kernel(Args a) {
  using C = ChainLay<D>;
  using SC = ChainSplitCols<D, CS>;
  constexpr int MD = C::MD, NP = C::NP, LDC = C::LDC, NX = 2 * D, NTH = 64 * SC::NW;
  constexpr int NPI = (D * D / 4 + NTH - 1) / NTH;   // float4 pieces of P per thread
  __shared__ __attribute__((aligned(16))) char smem[C::BYTES];
  const int wave = wave_id(), lane = threadIdx.x & 63, g = lane >> 4, cl = lane & 15;
  const int bh_ = blockIdx.x, b = bh_ / a.H, h = bh_ % a.H;
  const int cgrp = (int)blockIdx.y % SC::NH;                     // column group of this workgroup
  const int slot = a.slot0 + (int)blockIdx.y / SC::NH, dir = dir_of_slot(a.dirs, slot);
  const int mode = a.ch_mode;
  const int grp = mode == 1 ? (int)blockIdx.z >> 1 : (int)blockIdx.z;
  const bool pmul_only = mode == 1 && (blockIdx.z & 1) == 0;   // compose P: seed I, no Q
  const int strip = wave + SC::NW * cgrp;
  const bool act = strip < MD;                                   // wave-uniform
  const int col = 16 * (act ? strip : 0) + cl;
  const uint32_t so = (uint32_t)((4 * g * D + col) * 4);        // lane offset within a [D][D] state
  const uint32_t xq = (uint32_t)((col * NX + D + 4 * g) * 4);   // lane offset of Q^T within a [D][2D] map
  const uint32_t tso = (uint32_t)((col * D + 4 * g) * 4);       // lane offset within a transposed state
  const size_t hs = ((size_t)slot * a.B + b) * a.H + h;         // (slot, batch, head)
  // positions of this launch: [p0, p1) of the maps read (segment maps, or the group maps in mode 2)
  const int nsteps = a.NS - 1;
  const int p0 = (mode == 1 || mode == 3) ? grp * a.ch_m : 0;
  const int p1 = mode == 2 ? a.ch_groups : (mode == 1 || mode == 3) ? min(p0 + a.ch_m, nsteps) : nsteps;
  const float* maps = mode == 2 ? a.gmaps + hs * (size_t)a.ch_groups * D * NX : a.maps + hs * (size_t)a.NS * D * NX;
  // PT: the reversed scan of a bidirectional call, which takes P_p as the
  // transpose of the forward scan's P of the same segment (its Q half is its
  // own).  Never in mode 2 (group maps are stored in the plain layout).
  constexpr bool ptr = PT;
  const float* pmaps = ptr ? a.maps + ((size_t)b * a.H + h) * (size_t)a.NS * D * NX : maps;
  float* starts = mode == 2 ? a.gstarts + hs * (size_t)a.ch_groups * D * D : a.starts + hs * (size_t)a.NS * D * D;

  for (int i = threadIdx.x; i < C::BYTES / 16; i += NTH) reinterpret_cast<uint4*>(smem)[i] = make_uint4(0, 0, 0, 0);

  f32x4 H[MD];
  if (mode == 1) {
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) H[md][rr] = (pmul_only && 16 * md + 4 * g + rr == col) ? 1.f : 0.f;
  } else if (mode == 3) {
    const __amdgpu_buffer_rsrc_t r = block_rsrc(a.gstarts + (hs * a.ch_groups + grp) * (size_t)D * D, act ? D * D * 4 : 0);
#pragma unroll
    for (int md = 0; md < MD; ++md) H[md] = tile_load_t(r, tso, (uint32_t)(md * 16 * 4));
  } else {
    const float* seed = (dir == 0 || a.dirs == 2) ? a.h0 : nullptr;
    const __amdgpu_buffer_rsrc_t r =
        block_rsrc(seed ? seed + ((size_t)b * a.H + h) * D * D : a.starts, seed && act ? D * D * 4 : 0);
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) H[md][rr] = block_load(r, so, (uint32_t)((16 * md + rr) * D * 4));
  }
  // start states are stored in modes 0 and 3 (segment starts) and 2 (group starts)
  const bool store_starts = mode != 1 && act;
  const __amdgpu_buffer_rsrc_t st =
      block_rsrc(starts, store_starts ? (uint32_t)(mode == 2 ? a.ch_groups : a.NS) * D * D * 4 : 0);

  // Maps in flight, one step ahead: P (float4 number threadIdx.x + NTH i) and
  // Q (this lane's accumulator-layout tiles).
  typedef float4 PRegs[NPI];
  // Thread element f = threadIdx.x + NTH i holds row `row`, columns 4 c4 ..
  // 4 c4 + 3 of the staged P; transposed, those are one column of four rows
  // of the stored map (dword loads, coalesced along the column index).
  auto fetch_p = [&](int p, PRegs& r) {
    const __amdgpu_buffer_rsrc_t m = block_rsrc(pmaps + (size_t)(ptr ? a.NS - 1 - p : p) * D * NX, D * NX * 4);
    // pieces past the map (f >= D * D / 4) address past it: zeros
#pragma unroll
    for (int i = 0; i < NPI; ++i) {
      const int f = threadIdx.x + NTH * i;
      if constexpr (ptr) {
        const int row = f % D, c4 = f / D;
        r[i] = make_float4(block_load(m, (uint32_t)(((4 * c4 + 0) * NX + row) * 4), 0),
                           block_load(m, (uint32_t)(((4 * c4 + 1) * NX + row) * 4), 0),
                           block_load(m, (uint32_t)(((4 * c4 + 2) * NX + row) * 4), 0),
                           block_load(m, (uint32_t)(((4 * c4 + 3) * NX + row) * 4), 0));
      } else {
        const int row = f / (D / 4), c4 = f % (D / 4);
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(m, (uint32_t)((row * NX + 4 * c4) * 4), 0, 0);
        r[i] = __builtin_bit_cast(float4, v);
      }
    }
  };
  // Q of map p; compose-P reads none (an empty range: zeros)
  auto fetch_q = [&](int p, f32x4 (&q)[MD]) {
    const __amdgpu_buffer_rsrc_t m = block_rsrc(maps + (size_t)p * D * NX, pmul_only || !act ? 0 : D * NX * 4);
#pragma unroll
    for (int md = 0; md < MD; ++md) q[md] = tile_load_t(m, xq, (uint32_t)(16 * md * 4));
  };
  auto stage = [&](int buf, const PRegs& r) {
    bh* phi = reinterpret_cast<bh*>(smem + buf * 2 * C::MAT);
    bh* plo = phi + C::MAT / 2;
#pragma unroll
    for (int i = 0; i < NPI; ++i) {
      const int f = threadIdx.x + NTH * i;
      const int row = ptr ? f % D : f / (D / 4), c4 = ptr ? f / D : f % (D / 4);
      s16x4_t hi, lo;
      split4(f32x4{r[i].x, r[i].y, r[i].z, r[i].w}, hi, lo);
      if (NPI * NTH == D * D / 4 || f < D * D / 4) {
        *reinterpret_cast<s16x4_t*>(phi + row * LDC + 4 * c4) = hi;
        *reinterpret_cast<s16x4_t*>(plo + row * LDC + 4 * c4) = lo;
      }
    }
  };

  auto last = [&](int p) { return p < p1 ? p : p1 - 1; };   // clamped map index
  // P maps in flight: a whole chain (CS: one wavefront per SIMD, registers to
  // spare) fetches P two steps ahead, so that a map's loads have a step and a
  // half to arrive before it is staged; the split chain's launches one step
  // ahead.
  constexpr int AHEAD = CS ? 2 : 1;
  PRegs prA, prB;
  f32x4 qn[MD];   // Q of the current step's map, then of the next one
  // Step p: H_{p+1} = P_p H_p + Q_p with P_p staged in LDS buffer (p - p0) & 1;
  // P_{p+AHEAD} is fetched into `fetch_dst` meanwhile, and P_{p+1} (in
  // `stage_src`, fetched AHEAD - 1 steps earlier or meanwhile) is staged at
  // the end of the step.
  auto step = [&](int p, PRegs& stage_src, PRegs& fetch_dst) {
    // start state of position p (compose stores none: an empty range)
#pragma unroll
    for (int md = 0; md < MD; ++md) tile_store_t(st, tso, (uint32_t)((p * D * D + 16 * md) * 4), H[md]);
    s16x4_t hh[2 * NP], hl[2 * NP];
#pragma unroll
    for (int t = 0; t < 2 * NP; ++t) {
      if (t < MD) {
        split4(H[t], hh[t], hl[t]);
      } else {
        hh[t] = s16x4_t{0, 0, 0, 0};
        hl[t] = s16x4_t{0, 0, 0, 0};
      }
    }
    f32x4 acc[MD];
#pragma unroll
    for (int md = 0; md < MD; ++md) acc[md] = qn[md];
    fetch_q(last(p + 1), qn);
    fetch_p(last(p + AHEAD), fetch_dst);
    const bh* phi = reinterpret_cast<const bh*>(smem + ((p - p0) & 1) * 2 * C::MAT);
    const bh* plo = phi + C::MAT / 2;
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const bf16x8_t bhi = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(hh[2 * q], hh[2 * q + 1], 0, 1, 2, 3, 4, 5, 6, 7));
      const bf16x8_t blo = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(hl[2 * q], hl[2 * q + 1], 0, 1, 2, 3, 4, 5, 6, 7));
      // Tiles in groups of up to 4, each of the three products over the whole
      // group before the next: consecutive MFMAs update different
      // accumulators (three dependent ones in a row each wait for the last).
      constexpr int GRP = 4;
#pragma unroll
      for (int m0 = 0; m0 < MD; m0 += GRP) {
        bf16x8_t ahi[GRP], alo[GRP];
#pragma unroll
        for (int i = 0; i < GRP; ++i)
          if (m0 + i < MD) {
            ahi[i] = fragB2(phi + (16 * (m0 + i) + cl) * LDC, 2 * q, g);
            alo[i] = fragB2(plo + (16 * (m0 + i) + cl) * LDC, 2 * q, g);
          }
#pragma unroll
        for (int i = 0; i < GRP; ++i)
          if (m0 + i < MD) acc[m0 + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[i], bhi, acc[m0 + i], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < GRP; ++i)
          if (m0 + i < MD) acc[m0 + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[i], blo, acc[m0 + i], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < GRP; ++i)
          if (m0 + i < MD) acc[m0 + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[i], bhi, acc[m0 + i], 0, 0, 0);
      }
    }
#pragma unroll
    for (int md = 0; md < MD; ++md) H[md] = acc[md];
    stage((p + 1 - p0) & 1, stage_src);
    __syncthreads();
  };

  if (p1 > p0) {
    fetch_p(p0, prA);
    fetch_q(p0, qn);
    __syncthreads();   // zero fill done
    stage(0, prA);
    if constexpr (AHEAD == 2) fetch_p(last(p0 + 1), prA);
    __syncthreads();
  }
  // Drain the prologue's loads here, once: otherwise the wait the compiler
  // needs for the seed state on the loop's entry path is placed at the loop
  // header and executed every step, where it waits for the prefetched maps.
  __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
  if constexpr (AHEAD == 2) {
    // prA holds P_{p+1} at even offsets p - p0, prB at odd ones.  The loop
    // body has no branch (a step skipped on one path would leave its loads
    // pending at the loop header, where the compiler would then wait for
    // every load in flight); an odd last step runs after it.
    int p = p0;
    for (; p + 1 < p1; p += 2) {
      step(p, prA, prB);
      step(p + 1, prB, prA);
    }
    if (p < p1) step(p, prA, prB);
  } else {
    for (int p = p0; p < p1; ++p) step(p, prA, prA);
  }
  if (mode == 1) {
    // the group's map: P_g row-major, Q_g transposed
    const __amdgpu_buffer_rsrc_t xr = block_rsrc(a.gmaps + (hs * a.ch_groups + grp) * (size_t)D * NX, act ? D * NX * 4 : 0);
    if (pmul_only) {
      const uint32_t xo = (uint32_t)((4 * g * NX + col) * 4);
#pragma unroll
      for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int r = 0; r < 4; ++r) block_store(xr, xo, (uint32_t)((md * 16 + r) * NX * 4), H[md][r]);
    } else {
#pragma unroll
      for (int md = 0; md < MD; ++md) tile_store_t(xr, xq, (uint32_t)(md * 16 * 4), H[md]);
    }
  } else if (mode == 0 || (mode == 3 && p1 == nsteps)) {
    // the final state of the chain, at position NS - 1
#pragma unroll
    for (int md = 0; md < MD; ++md) tile_store_t(st, tso, (uint32_t)(((a.NS - 1) * D * D + 16 * md) * 4), H[md]);
  }
}

// ---------------------------------------------------------------------------
// 3. Outputs.  grid (segments padded to a multiple of 8, B * H), one launch
// per scan direction: each workgroup re-runs its segment from the start state
// of the chain (or, for the chunk-causal reversed scan, a chunk of frames from
// zero).  Mode 1 stores the outputs as an fp16 partial, mode 2 adds the
// partial before the single final store (bidirectional: the forward launch
// stores, the reversed one adds; chunk-causal: the other way round).  Strip
// wave w owns state columns 16 w .. 16 w + 15.
template <int D, bool PRO, int ST, bool TML>
__global__ __launch_bounds__(Geo<D>::NT) void seg_out_kernel(Args a) {
  using G = Geo<D>;
  using L = Lay<D, true>;
  constexpr int MD = G::MD, SPW = 1;
  // TML: the Tm blocks come from the map kernel of this scan; the helper
  // stages them and forms most of the P tiles instead of inverting I + A.
  constexpr int HP = kHelperP(G::NSW), SP = 10 - HP;   // P tiles of the helper, of the strips
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
  const int wave = wave_id(), lane = threadIdx.x & 63, g = lane >> 4, cl = lane & 15;
  const int seg = blockIdx.x;
  if (seg >= a.npos) return;                        // padding of the grid (whole workgroup)
  const int bh_ = a.heads_rev ? (int)(gridDim.y - 1 - blockIdx.y) : (int)blockIdx.y, b = bh_ / a.H, h = bh_ % a.H;
  // A segment is L tokens whose start state the chain computed, or (the
  // chunk-causal reversed scan) one chunk of frames, started from zero.
  const bool chunks = a.cs_len > 0;
  const long long s0 = !chunks ? (long long)seg * a.L : seg == 0 ? 0 : a.cs_first + (long long)(seg - 1) * a.cs_len;
  const long long e0 = !chunks ? s0 + a.L : seg == 0 ? a.cs_first : s0 + a.cs_len;
  const long long s1 = e0 < a.T ? e0 : a.T;
  const int nsub = (int)((s1 - s0 + CH - 1) / CH);
  const size_t sbase = ((size_t)b * a.H + h) * D * D;
  const Inv I = inv_at<D, true>(smem);
  const bool helper = wave == G::HW;
  const int col = 16 * wave + cl;                  // state / value column of a strip lane
  const long long HD = (long long)a.H * D;
  const uint32_t so = (uint32_t)((4 * g * D + col) * 4);   // lane byte offset within a state

  for (int i = threadIdx.x; i < L::BYTES / 16; i += G::NT) reinterpret_cast<uint4*>(smem)[i] = make_uint4(0, 0, 0, 0);

  {
    const int dir = a.dir;
    const bool rev = dir == 1;
    const int slot = slot_of_dir(a.dirs, dir);
    const int pos = rev ? a.NS - 1 - seg : seg;
    f32x4 H[SPW][MD];
    if (!helper && chunks) {
#pragma unroll
      for (int md = 0; md < MD; ++md) H[0][md] = zero4();
    } else if (!helper) {
      const float* stp = a.starts + ((((size_t)slot * a.B + b) * a.H + h) * a.NS + pos) * (size_t)D * D;
      const __amdgpu_buffer_rsrc_t hr = block_rsrc(stp, D * D * 4);
      const uint32_t tso = (uint32_t)((col * D + 4 * g) * 4);   // starts are transposed
#pragma unroll
      for (int md = 0; md < MD; ++md) H[0][md] = tile_load_t(hr, tso, (uint32_t)(md * 16 * 4));
    }
    auto piece = [&](int jj) {   // sub-chunk jj of the scan; past the segment: empty
      const int jc = rev ? nsub - 1 - jj : jj;
      const long long t0 = jj < nsub ? s0 + (long long)jc * CH : s0;
      return make_sub(t0, jj < nsub ? (int)((s1 - t0) < CH ? (s1 - t0) : CH) : 0, rev);
    };
    StageKQ sk;
    StageV sv;
    StageG sg;
    StageTm stm;
    {
      const Sub s0b = piece(0), s1b = piece(1);
      if (helper) {
        fetch_gates(a, b, h, s0b, sg);
        if constexpr (TML) fetch_tm(tm_rsrc(a, slot, b, h, s0b), stm);
      } else {
        fetch_kq<D, true, PRO>(a, b, h, s0b, sk);
        fetch_v<D>(a, b, h, s0b, sv);
      }
      __syncthreads();
      if (helper) {
        stage_gates(buf_at<D, true>(smem, 0), sg, a.c);
        fetch_gates(a, b, h, s1b, sg);
        if constexpr (TML) {
          stage_tm(buf_at<D, true>(smem, 0), stm);
          fetch_tm(tm_rsrc(a, slot, b, h, s1b), stm);
        }
      } else {
        stage_kq<D, true, PRO>(buf_at<D, true>(smem, 0), sk);
        stage_v<D>(buf_at<D, true>(smem, 0), sv);
        fetch_kq<D, true, PRO>(a, b, h, s1b, sk);
        fetch_v<D>(a, b, h, s1b, sv);
      }
      __syncthreads();
      if constexpr (TML) {
        if (helper) gram_p_tiles<D, HP>(a, buf_at<D, true>(smem, 0), SP, 1);
        else gram_p_tiles<D, 1>(a, buf_at<D, true>(smem, 0), wave < SP ? wave : 10, 0);
      } else {
        if (helper) gram_stage_helper<D>(a, buf_at<D, true>(smem, 0), I);
        else gram_stage_strips<D, true>(a, buf_at<D, true>(smem, 0), I);
      }
      __syncthreads();
    }
    if (helper) {
      // helper: gate factors of c+1, and either the inverse of c and the
      // diagonal A blocks of c+1, or (TML) c+1's Tm blocks and P tiles
      for (int c = 0; c < nsub; ++c) {
        const Buf Bc = buf_at<D, true>(smem, c & 1), Bn = buf_at<D, true>(smem, (c + 1) & 1);
        const Inv I = inv_at<D, true>(smem);
        stage_gates(Bn, sg, a.c);
        fetch_gates(a, b, h, piece(c + 2), sg);
        if constexpr (TML) {
          stage_tm(Bn, stm);
          fetch_tm(tm_rsrc(a, slot, b, h, piece(c + 2)), stm);
        } else {
          tinv_offdiag(I, Bc);
        }
        __syncthreads();
        if constexpr (TML) {
          if (c + 1 < nsub) gram_p_tiles<D, HP>(a, Bn, SP, 1);
        } else {
          if (c + 1 < nsub) gram_stage_helper<D>(a, Bn, I);
        }
        __syncthreads();
      }
      return;
    }
    // Outputs.  Sub-chunk c's tiles are written to the staging rows at the end
    // of beta c and stored from there in alpha c+1 as whole rows (each thread
    // 4 x 4 consecutive values), so that global stores and partial loads cover
    // whole cache lines instead of each strip's 64-byte share of a row.  In
    // mode 2 the partial is added there, loaded in the same row layout one
    // sub-chunk ahead.
    constexpr int NTS = 64 * G::NSW, C4 = D / 4;   // strip threads; 4-column groups per row
    static_assert(CH * C4 == 4 * NTS, "four groups of four values per strip thread");
    const int t = threadIdx.x;
    // ST: what this launch stores, a template parameter so that every store
    // is unconditional (stores behind a branch make the compiler assume they
    // may not have been issued and wait for later stores where it waits for
    // earlier loads): 0 fp32 outputs, 1 bf16 outputs, 2 the fp16 partial of
    // mode 1 (half the bytes of fp32 each way; it adds a rounding of 2^-11 of
    // the partial's magnitude to the sum), 3 and 4: fp32 and bf16 outputs
    // with the partial added (mode 2; only these load it).
    constexpr bool ADD = ST >= 3;
    constexpr int SO = ADD ? ST - 3 : ST;
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    const long long esz = SO == 0 ? 4 : 2;
    char* const dstb = static_cast<char*>(SO == 2 ? static_cast<void*>(a.part) : a.out);
    u32x2_t pre[4] = {u32x2_t{0u, 0u}, u32x2_t{0u, 0u}, u32x2_t{0u, 0u}, u32x2_t{0u, 0u}};   // fp16 partial
    auto rows_of = [&](int c) { return ((long long)b * a.T + piece(c).t0) * HD + (long long)h * D; };
    auto load_pre = [&](int c) {
      if constexpr (!ADD) return;
      const Sub sb = piece(c);
      const __amdgpu_buffer_rsrc_t rs = rows_rsrc(a.part + rows_of(c), (long long)sb.n * HD * 2);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = t + NTS * i, row = k / C4, c4 = k % C4;
        pre[i] = __builtin_amdgcn_raw_buffer_load_b64(rs, (uint32_t)(((sb.r0 + sb.sgn * row) * (int)HD + 4 * c4) * 2), 0, 0);
      }
    };
    auto pre_f32 = [](u32x2_t w) {
      return f32x4{(float)__builtin_bit_cast(_Float16, (uint16_t)(w[0] & 0xffffu)),
                   (float)__builtin_bit_cast(_Float16, (uint16_t)(w[0] >> 16)),
                   (float)__builtin_bit_cast(_Float16, (uint16_t)(w[1] & 0xffffu)),
                   (float)__builtin_bit_cast(_Float16, (uint16_t)(w[1] >> 16))};
    };
    // Store the staged outputs of sub-chunk c (rows past n fall outside the
    // buffer).  c = -1 stores nothing (an empty range) but issues the same
    // stores, so that every iteration issues the same memory operations and
    // the compiler's wait counts stay exact (a skipped flush in the first
    // iteration made it wait for the stores of every later one).
    auto flush = [&](int c) {
      const Sub sb = piece(c < 0 ? 0 : c);
      const Inv I = inv_at<D, true>(smem);
      const __amdgpu_buffer_rsrc_t rs =
          rows_rsrc(dstb + rows_of(c < 0 ? 0 : c) * esz, c < 0 ? 0 : (long long)sb.n * HD * esz);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = t + NTS * i, row = k / C4, c4 = k % C4;
        f32x4 val = ld4f(I.os + row * L::OSL + 4 * c4);
        if constexpr (ADD) val = val + pre_f32(pre[i]);
        const uint32_t off = (uint32_t)(((sb.r0 + sb.sgn * row) * (int)HD + 4 * c4) * esz);
        if constexpr (SO == 1) {
          const u32x2_t w{f32_to_bf16_bits(val[0]) | ((uint32_t)f32_to_bf16_bits(val[1]) << 16),
                          f32_to_bf16_bits(val[2]) | ((uint32_t)f32_to_bf16_bits(val[3]) << 16)};
          __builtin_amdgcn_raw_buffer_store_b64(w, rs, off, 0, 0);
        } else if constexpr (SO == 2) {
          const u32x2_t w{(uint32_t)f2h(val[0]) | ((uint32_t)f2h(val[1]) << 16),
                          (uint32_t)f2h(val[2]) | ((uint32_t)f2h(val[3]) << 16)};
          __builtin_amdgcn_raw_buffer_store_b64(w, rs, off, 0, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, val), rs, off, 0, 0);
        }
      }
    };
    f32x4 R[SPW][4];
    for (int c = 0; c < nsub; ++c) {
      const Buf Bc = buf_at<D, true>(smem, c & 1), Bn = buf_at<D, true>(smem, (c + 1) & 1);
      const Inv I = inv_at<D, true>(smem);
      // alpha.  Staging first: it waits for the prefetched rows, which were
      // issued before the stores and loads below (the load counter drains in
      // issue order).  The K/Q rows of c+2 are requested in beta, after the
      // first products (measured 2% faster than here: alpha's memory
      // instructions queue behind the stores).
      stage_kq<D, true, PRO>(Bn, sk);
      flush(c - 1);
      load_pre(c);
      {
        f16x8_t Hp[SPW][G::NP];
        state_pairs<D>(H[0], Hp[0]);
        wrows_state<D, SPW, false>(Bc.kr, Hp, cl, g, R);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          R[0][mt] = vals_tile<D>(Bc.vr, mt, wave, cl, g) - ld4f(Bc.ce + 16 * mt + 4 * g) * R[0][mt];
      }
      __syncthreads();
      // beta: the V rows of c+1 replace those of c (read in alpha only)
      stage_v<D>(Bc, sv);
      fetch_v<D>(a, b, h, piece(c + 2), sv);
      {
        f32x4 O[1][4];   // outputs, transposed tiles (lane: token 16 mt + cl, columns 4g ..)
        {
          f16x8_t Hp[1][G::NP];
          state_pairs<D>(H[0], Hp[0]);
          wrows_state<D, 1, true>(Bc.qr, Hp, cl, g, O);
        }
        fetch_kq<D, true, PRO>(a, b, h, piece(c + 2), sk);
        f16x8_t Rh[SPW][2];
        Rh[0][0] = tof16x8(R[0][0], R[0][1]);
        Rh[0][1] = tof16x8(R[0][2], R[0][3]);
        f32x4 Vn[SPW][4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) Vn[0][mt] = zero4();
        wtri<SPW, false>(Bc.tt, Rh, cl, g, Vn);
        f16x8_t Vh[SPW][2];
        Vh[0][0] = tof16x8(Vn[0][0], Vn[0][1]);
        Vh[0][1] = tof16x8(Vn[0][2], Vn[0][3]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) O[0][mt] = Bc.eg[16 * mt + cl] * O[0][mt];
        wtri<1, true>(Bc.pp, Vh, cl, g, O);
        f16x8_t Vs[SPW][2];
        const f32x4 d0 = ld4f(Bc.dn + 4 * g), d1 = ld4f(Bc.dn + 16 + 4 * g);
        const f32x4 d2 = ld4f(Bc.dn + 32 + 4 * g), d3 = ld4f(Bc.dn + 48 + 4 * g);
        Vs[0][0] = tof16x8(Vn[0][0] * d0, Vn[0][1] * d1);
        Vs[0][1] = tof16x8(Vn[0][2] * d2, Vn[0][3] * d3);
        wstate_update<D, SPW>(Bc.kr, Vs, Bc.eg[CH - 1], cl, g, H);
        // The Gram products of c+1, then the output staging, then the Gram
        // epilogues: every LDS read of the phase is placed before its first
        // LDS store, which it would otherwise wait behind.
        const bool more = c + 1 < nsub;
        f32x4 skp[1];
        f32x4 sks[GramStrips<D, true>::NK];
        if constexpr (TML) {
          if (more) gram_p_products<D, 1>(Bn, wave < SP ? wave : 10, 0, skp);
        } else {
          if (more) gram_strips_products<D, true>(Bn, sks);
        }
        // staging rows: row 16 mt + cl, columns 16 wave + 4 g ..
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          *reinterpret_cast<f32x4*>(I.os + (16 * mt + cl) * L::OSL + 16 * wave + 4 * g) = O[0][mt];
        if constexpr (TML) {
          if (more) gram_p_epilogues<1>(a, Bn, wave < SP ? wave : 10, 0, skp);
        } else {
          if (more) gram_strips_epilogues<D, true>(a, Bn, I, sks);
        }
      }
      __syncthreads();
    }
    if (nsub > 0) flush(nsub - 1);
    // final state: the scan's last segment
    if (a.hT && !chunks && pos == a.NS - 1 && (dir == 0 || a.dirs == 2)) {
      const __amdgpu_buffer_rsrc_t hr = block_rsrc(a.hT + sbase, D * D * 4);
#pragma unroll
      for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int r = 0; r < 4; ++r) block_store(hr, so, (uint32_t)((md * 16 + r) * D * 4), H[0][md][r]);
    }
  }
}

// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// 4. Frame-level (Jacobi) transition.  [WM-summary] section 3.2, frame-wise
// update: every token of a frame reads the frame's end state, and the frame
// maps the state as H_end = gamma (I - c^2 K^T diag(beta) K) H + c K^T diag(beta) V
// (one decay per frame: the gate of the frame's first token in the scan
// order).  The per-frame maps are independent, the chain composes them over
// the frames (the same kernel as above, with one "segment" per frame), and the
// outputs of a frame are one product Q H_end; in a bidirectional call
// O = Q (H_end^fwd + H_end^rev), the output being linear in the state.

// Rows of one 64-token piece in the staging thread mapping (two rows and 8
// components per thread): K, V and per-row beta.
struct JacStage {
  uint4 k[2], v[2];
  float b[2], fk[2];   // beta and (feature prologue) key factor of the rows
};

template <int D, bool PRO>
__device__ __forceinline__ void jac_fetch(const Args& a, int b, int h, long long t0, int n, JacStage& st) {
  const int t = threadIdx.x, i2 = t / (D / 8), c8 = t % (D / 8);
  const int HD = a.H * D;
  const long long e0 = ((long long)b * a.T + t0) * HD + (long long)h * D;
  const __amdgpu_buffer_rsrc_t rk = rows_rsrc(a.k + e0, (long long)n * HD * 2);
  const __amdgpu_buffer_rsrc_t rv = rows_rsrc(a.v + e0, (long long)n * HD * 2);
  const __amdgpu_buffer_rsrc_t rb = rows_rsrc(a.beta + ((long long)b * a.T + t0) * a.H + h, (long long)n * a.H * 4);
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int row = 2 * i2 + r;
    const uint32_t off = (uint32_t)(row * HD * 2 + 16 * c8);
    st.k[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
    st.v[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
    st.b[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, (uint32_t)(row * a.H * 4), 0, 0));
  }
  if constexpr (PRO) {
    const f32x4 f = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  fac_rsrc(a, b, h, t0), (uint32_t)((2 * i2 + 1) * 8), 0, 0));
    st.fk[0] = f[0];
    st.fk[1] = f[2];
  }
}

// LDS of the map kernel: two buffers of K, c^2 beta K and c beta V rows (fp16,
// the K-row layout above).
template <int D>
struct JacLay {
  static constexpr int MAT = (KRows<D>::ELEMS * 2 + 15) / 16 * 16;
  static constexpr int BUF = 3 * MAT;
  static constexpr int BYTES = 2 * BUF;
  static_assert(BYTES <= 160 * 1024, "workgroup LDS budget exceeded");
};

// grid (F, B * H), D/16 wavefronts: wave w accumulates column strip w of
// M = c^2 K^T diag(beta) K and of N = c K^T diag(beta) V over the frame's
// tokens, 64 at a time; both MFMA operands are transposing reads of the staged
// rows (contraction over tokens, in the register-B token order).
template <int D, bool PRO>
__global__ __launch_bounds__(64 * (D / 16)) void jac_map_kernel(Args a) {
  using J = JacLay<D>;
  constexpr int MD = D / 16;
  __shared__ __attribute__((aligned(16))) char smem[J::BYTES];
  const int wave = wave_id(), lane = threadIdx.x & 63, g = lane >> 4, cl = lane & 15;
  const int f = blockIdx.x, bh_ = blockIdx.y, b = bh_ / a.H, h = bh_ % a.H;
  const int S = a.L, F = a.NS - 1;
  const long long tf = (long long)f * S;
  const int np = (S + CH - 1) / CH;
  const float c = a.c;
  for (int i = threadIdx.x; i < J::BYTES / 16; i += 64 * MD) reinterpret_cast<uint4*>(smem)[i] = make_uint4(0, 0, 0, 0);
  auto piece_n = [&](int p) { return p < np ? (S - CH * p < CH ? S - CH * p : CH) : 0; };
  auto stage = [&](int buf, const JacStage& st) {
    hb* kr = reinterpret_cast<hb*>(lds_at(smem, (uint32_t)(buf * J::BUF)));
    hb* bk = kr + J::MAT / 2;
    hb* bv = bk + J::MAT / 2;
    const int t = threadIdx.x, i2 = t / (D / 8), c8 = t % (D / 8);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int o = krow<D>(2 * i2 + r) + 8 * c8;
      // PRO: key features ReLU(f_k k); the factor is positive, so the ReLU
      // of the scaled row is the scaled ReLU
      const float fk = PRO ? st.fk[r] : 1.f;
      *reinterpret_cast<uint4*>(kr + o) = PRO ? bf16x8_scaled_f16x8<true>(st.k[r], fk) : bf16x8_to_f16x8(st.k[r]);
      *reinterpret_cast<uint4*>(bk + o) = bf16x8_scaled_f16x8<PRO>(st.k[r], c * c * st.b[r] * fk);
      *reinterpret_cast<uint4*>(bv + o) = bf16x8_scaled_f16x8<false>(st.v[r], c * st.b[r]);
    }
  };
  f32x4 acc[MD][2];
#pragma unroll
  for (int md = 0; md < MD; ++md) acc[md][0] = acc[md][1] = zero4();
  JacStage st;
  jac_fetch<D, PRO>(a, b, h, tf, piece_n(0), st);
  __syncthreads();   // zero fill done
  stage(0, st);
  jac_fetch<D, PRO>(a, b, h, tf + CH, piece_n(1), st);
  __syncthreads();
  // lane (g, a + 4 j) addresses row 4 g + j, columns 4 a .. of a 16-column block
  const int toff = krow<D>(4 * g + (cl >> 2)) + 4 * (cl & 3);
  for (int p = 0; p < np; ++p) {
    const hb* kr = reinterpret_cast<const hb*>(lds_at(smem, (uint32_t)((p & 1) * J::BUF))) + toff;
    const hb* bk = kr + J::MAT / 2;
    const hb* bv = bk + J::MAT / 2;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int r0 = krow<D>(32 * q), r1 = krow<D>(32 * q + 16);
      const f16x8_t xm = cat8(ld4_tr(bk + r0 + 16 * wave), ld4_tr(bk + r1 + 16 * wave));
      const f16x8_t xn = cat8(ld4_tr(bv + r0 + 16 * wave), ld4_tr(bv + r1 + 16 * wave));
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        const f16x8_t at = cat8(ld4_tr(kr + r0 + 16 * md), ld4_tr(kr + r1 + 16 * md));
        acc[md][0] = mfma32(at, xm, acc[md][0]);
        acc[md][1] = mfma32(at, xn, acc[md][1]);
      }
    }
    if (p + 1 < np) stage((p + 1) & 1, st);
    jac_fetch<D, PRO>(a, b, h, tf + (long long)CH * (p + 2), piece_n(p + 2), st);
    __syncthreads();
  }
  // maps: forward scan (position f, decay of the frame's first token) and
  // reversed scan (position F-1-f, decay of its last token)
  const int col = 16 * wave + cl;
  const uint32_t xo = (uint32_t)((4 * g * 2 * D + col) * 4);
  const float* gg = a.g + ((long long)b * a.T + tf) * a.H + h;
#pragma unroll
  for (int dir = 0; dir < 2; ++dir) {
    if (!(a.dirs & (1 << dir))) continue;
    const int slot = slot_of_dir(a.dirs, dir);
    const int pos = dir == 0 ? f : F - 1 - f;
    const float gam = expf(gg[(long long)(dir == 0 ? 0 : S - 1) * a.H]);
    const float* Xg = a.maps + ((((size_t)slot * a.B + b) * a.H + h) * a.NS + pos) * (size_t)D * (2 * D);
    const __amdgpu_buffer_rsrc_t xr = block_rsrc(Xg, D * 2 * D * 4);
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * md + 4 * g + r;   // the lane offset xo holds the 4 g rows
        block_store(xr, xo, (uint32_t)((16 * md + r) * 2 * D * 4), gam * ((row == col ? 1.f : 0.f) - acc[md][0][r]));
      }
    const uint32_t xq = (uint32_t)((col * 2 * D + D + 4 * g) * 4);   // Q^T
#pragma unroll
    for (int md = 0; md < MD; ++md) tile_store_t(xr, xq, (uint32_t)(md * 16 * 4), acc[md][1]);
  }
}

// Outputs: grid (F, B * H), D/16 wavefronts; wave w owns output columns
// 16 w .. 16 w + 15.  The frame's end state (summed over the scans present) is
// split into fp16 hi + lo parts (about 22 significant bits) and each 64-row
// piece of Q is multiplied by both.
template <int D, bool PRO, bool OB>
__global__ __launch_bounds__(64 * (D / 16)) void jac_out_kernel(Args a) {
  using G = Geo<D>;
  constexpr int MD = D / 16;
  constexpr int MAT = (KRows<D>::ELEMS * 2 + 15) / 16 * 16;
  // output staging: 64 rows of D fp32 values, OSL floats apart, so that the
  // global stores cover whole rows (whole cache lines) instead of each strip
  // wave's 64-byte share of a row
  constexpr int OSL = D + 4, C4 = D / 4, NTH = 64 * (D / 16);
  static_assert(CH * C4 == 4 * NTH, "four groups of four values per thread");
  __shared__ __attribute__((aligned(16))) char smem[2 * MAT + CH * OSL * 4];
  const int wave = wave_id(), lane = threadIdx.x & 63, g = lane >> 4, cl = lane & 15;
  const int f = blockIdx.x, bh_ = blockIdx.y, b = bh_ / a.H, h = bh_ % a.H;
  const int S = a.L, F = a.NS - 1;
  const long long tf = (long long)f * S;
  const int np = (S + CH - 1) / CH;
  const int col = 16 * wave + cl;
  const uint32_t so = (uint32_t)((4 * g * D + col) * 4);
  const uint32_t tso = (uint32_t)((col * D + 4 * g) * 4);   // starts are transposed
  const long long HD = (long long)a.H * D;
  for (int i = threadIdx.x; i < 2 * MAT / 16; i += 64 * MD) reinterpret_cast<uint4*>(smem)[i] = make_uint4(0, 0, 0, 0);
  float* const os = reinterpret_cast<float*>(lds_at(smem, (uint32_t)(2 * MAT)));
  f32x4 Hs[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) Hs[md] = zero4();
#pragma unroll
  for (int dir = 0; dir < 2; ++dir) {
    if (!(a.dirs & (1 << dir))) continue;
    const int slot = slot_of_dir(a.dirs, dir);
    const int pos_end = dir == 0 ? f + 1 : F - f;
    const float* sp = a.starts + ((((size_t)slot * a.B + b) * a.H + h) * a.NS + pos_end) * (size_t)D * D;
    const __amdgpu_buffer_rsrc_t hr = block_rsrc(sp, D * D * 4);
#pragma unroll
    for (int md = 0; md < MD; ++md) Hs[md] += tile_load_t(hr, tso, (uint32_t)(md * 16 * 4));
  }
  // final state of the scan reported (forward when present), from its last position
  if (f == 0 && a.hT) {
    const float* sp = a.starts + (((size_t)b * a.H + h) * a.NS + F) * (size_t)D * D;
    const __amdgpu_buffer_rsrc_t hr = block_rsrc(sp, D * D * 4);
    const __amdgpu_buffer_rsrc_t tr = block_rsrc(a.hT + ((size_t)b * a.H + h) * D * D, D * D * 4);
#pragma unroll
    for (int md = 0; md < MD; ++md) {
      const f32x4 v = tile_load_t(hr, tso, (uint32_t)(md * 16 * 4));
#pragma unroll
      for (int r = 0; r < 4; ++r) block_store(tr, so, (uint32_t)((md * 16 + r) * D * 4), v[r]);
    }
  }
  f32x4 Hl[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) {
    const f16x4_t hi = tof16(Hs[md]);
    Hl[md] = Hs[md] - f32x4{(float)hi[0], (float)hi[1], (float)hi[2], (float)hi[3]};
  }
  f16x8_t Ph[G::NP], Pl[G::NP];
  state_pairs<D>(Hs, Ph);
  state_pairs<D>(Hl, Pl);
  // Q rows: thread (i2, c8) holds rows 2 i2, 2 i2 + 1, components 8 c8 ..
  const int t = threadIdx.x, i2 = t / (D / 8), c8 = t % (D / 8);
  auto piece_n = [&](int p) { return p < np ? (S - CH * p < CH ? S - CH * p : CH) : 0; };
  // PRO: the query factors of the two rows ride along in fq
  float fq[2] = {1.f, 1.f};
  auto fetch = [&](int p, uint4 (&qv)[2]) {
    const __amdgpu_buffer_rsrc_t rq = rows_rsrc(a.q + ((long long)b * a.T + tf + CH * p) * HD + (long long)h * D,
                                                (long long)piece_n(p) * HD * 2);
#pragma unroll
    for (int r = 0; r < 2; ++r)
      qv[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rq, (uint32_t)((2 * i2 + r) * HD * 2 + 16 * c8), 0, 0));
    if constexpr (PRO) {
      const f32x4 f = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    fac_rsrc(a, b, h, tf + CH * p), (uint32_t)((2 * i2 + 1) * 8), 0, 0));
      fq[0] = f[1];
      fq[1] = f[3];
    }
  };
  auto stage = [&](int buf, const uint4 (&qv)[2]) {
    hb* qr = reinterpret_cast<hb*>(lds_at(smem, (uint32_t)(buf * MAT)));
#pragma unroll
    for (int r = 0; r < 2; ++r)
      *reinterpret_cast<uint4*>(qr + krow<D>(2 * i2 + r) + 8 * c8) =
          PRO ? bf16x8_scaled_f16x8<false>(qv[r], fq[r]) : bf16x8_to_f16x8(qv[r]);
  };
  uint4 qv[2];
  fetch(0, qv);
  __syncthreads();   // zero fill done
  stage(0, qv);
  fetch(1, qv);
  __syncthreads();
  constexpr bool half = OB;   // bf16 outputs; a template parameter so the stores are unconditional
  const long long esz = half ? 2 : 4;
  for (int p = 0; p < np; ++p) {
    const hb* qr = reinterpret_cast<const hb*>(lds_at(smem, (uint32_t)((p & 1) * MAT)));
    f32x4 O[4], Ol[4];
    state_times_rows_T<D>(qr, Ph, cl, g, O);
    state_times_rows_T<D>(qr, Pl, cl, g, Ol);
    // staging rows: row 16 mt + cl, columns 16 wave + 4 g ..
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) *reinterpret_cast<f32x4*>(os + (16 * mt + cl) * OSL + 16 * wave + 4 * g) = O[mt] + Ol[mt];
    __syncthreads();
    // whole rows: thread t stores four pieces of four consecutive values (rows
    // past the piece fall outside the buffer)
    const long long rowb = ((long long)b * a.T + tf + CH * p) * HD + (long long)h * D;
    const __amdgpu_buffer_rsrc_t rs =
        rows_rsrc(static_cast<char*>(a.out) + rowb * esz, (long long)piece_n(p) * HD * esz);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = t + NTH * i, row = k / C4, c4 = k % C4;
      const f32x4 val = ld4f(os + row * OSL + 4 * c4);
      const uint32_t off = (uint32_t)((row * (int)HD + 4 * c4) * esz);
      if constexpr (half) {
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        const u32x2_t w{f32_to_bf16_bits(val[0]) | ((uint32_t)f32_to_bf16_bits(val[1]) << 16),
                        f32_to_bf16_bits(val[2]) | ((uint32_t)f32_to_bf16_bits(val[3]) << 16)};
        __builtin_amdgcn_raw_buffer_store_b64(w, rs, off, 0, 0);
      } else {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, val), rs, off, 0, 0);
      }
    }
    if (p + 1 < np) stage((p + 1) & 1, qv);
    fetch(p + 2, qv);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// 5. Strip scan: short single-direction calls (one streaming frame).
//
// With few sub-chunks per head the segment maps and the chain are mostly
// fixed latency (three launches, each about one sub-chunk long plus its ramp),
// and a head's sub-chunks in sequence would be one workgroup's long chain.
// But each column of the state evolves on its own (the update mixes rows
// through k and beta, never columns), so the sequence can be split by value
// columns instead of by tokens:
//   sc_prep_kernel (one workgroup per sub-chunk and head, all in parallel):
//     gate factors, the Gram tiles and the triangular inverse of the sub-chunk,
//     stored as Tm diag(beta) and P = c tril(Q K^T) * E (fp16, the 10 lower
//     16x16 blocks each) and the factors e^G, c e^G, c e^{G_n - G};
//   sc_scan_kernel (one workgroup per 16-column strip of the state and head):
//     the sub-chunks in scan order with short dependent steps.  Four compute
//     wavefronts, wave r owning the outputs of 16-token row tile r and state
//     tiles r and r + 4, each form in registers
//       K H (all 64 rows) and (Q H)^T (its rows)   (the state strip from LDS, fp16)
//       R = V - c e^G * K H,  V' = Tm diag(beta) R (all 64 rows)
//       O = e^G * Q H + P V'               -> global (its rows)
//       H <- e^{G_n} H + K^T (c e^{G_n - G} V')   (its state tiles -> LDS)
//     with one barrier per sub-chunk (the state strip double-buffered in LDS);
//     four stager wavefronts convert and stage the next sub-chunk's rows
//     meanwhile, their loads issued two sub-chunks ahead.  The same algebra
//     and rounding points as the output kernel, in another order of the sums.
// Measured on one 880-token frame of 20 heads x 112 (the streaming shape):
// 60 -> 31 us a call (captured in a HIP graph).  Each wave repeating K H and
// V' for the whole strip (16 and 6 products instead of 4 and 1-2) removed
// the exchanges of R and V' through LDS and two of three barriers per
// sub-chunk: the scan kernel 27.9 -> 24.2 us.  Staging (bf16 -> fp16
// conversion and scattered LDS writes) cost about 9 us of the three-barrier
// kernel's 27 (a copy without it ran in 18 us); preparing the rows in fp16
// in the prep kernel instead measured no faster (prep 11 -> 15 us, scan
// 27 -> 25.5 us).

// Per sub-chunk and head in the workspace: Tm diag(beta) and P as 320 pieces
// of 16 bytes each (the piece order of the stored inverses), then e^G,
// c e^G and c e^{G_n - G} (64 floats each).
constexpr int kScanSubBytes = 2 * kTmPieces * 16 + 3 * CH * 4;

template <int D>
struct PrepLay {
  static constexpr int KR = (KRows<D>::ELEMS * 2 + 15) / 16 * 16;
  static constexpr int o_qr = 0, o_kr = KR, o_pp = 2 * KR, o_tt = o_pp + CH * LDT * 2, o_gt = o_tt + CH * LDT * 2;
  static constexpr int o_ao = o_gt + 5 * CH * 4, o_td = o_ao + CH * LDT * 2, o_ad = o_td + CH * LDD * 2;
  static constexpr int BYTES = o_ad + 4 * ADB * 4;
};

template <int D>
__global__ __launch_bounds__(Geo<D>::NT) void sc_prep_kernel(Args a) {
  using G = Geo<D>;
  using PL = PrepLay<D>;
  __shared__ __attribute__((aligned(16))) char smem[PL::BYTES];
  const long long U = (a.T + CH - 1) / CH;
  const int jc = blockIdx.x;   // sub-chunk in original order
  if (jc >= U) return;
  const int b = (int)blockIdx.y / a.H, h = (int)blockIdx.y % a.H;
  const bool helper = wave_id() == G::HW;
  const long long t0 = (long long)jc * CH;
  const Sub sb = make_sub(t0, (int)(a.T - t0 < CH ? a.T - t0 : CH), a.dir == 1);
  Buf B;
  B.qr = reinterpret_cast<hb*>(smem + PL::o_qr);
  B.kr = reinterpret_cast<hb*>(smem + PL::o_kr);
  B.pp = reinterpret_cast<hb*>(smem + PL::o_pp);
  B.tt = reinterpret_cast<hb*>(smem + PL::o_tt);
  B.vr = nullptr;
  float* gt = reinterpret_cast<float*>(smem + PL::o_gt);
  B.g2 = gt;
  B.eg = gt + CH;
  B.ce = gt + 2 * CH;
  B.dn = gt + 3 * CH;
  B.bt = gt + 4 * CH;
  Inv I;
  I.ao = reinterpret_cast<hb*>(smem + PL::o_ao);
  I.td = reinterpret_cast<hb*>(smem + PL::o_td);
  I.ad = reinterpret_cast<float*>(smem + PL::o_ad);
  I.os = nullptr;
  for (int i = threadIdx.x; i < PL::BYTES / 16; i += G::NT) reinterpret_cast<uint4*>(smem)[i] = make_uint4(0, 0, 0, 0);
  StageG sg;
  StageKQ sk;
  if (helper)
    fetch_gates(a, b, h, sb, sg);
  else
    fetch_kq<D, true, false>(a, b, h, sb, sk);
  __syncthreads();
  if (helper)
    stage_gates(B, sg, a.c);
  else
    stage_kq<D, true, false>(B, sk);
  __syncthreads();
  if (helper)
    gram_stage_helper<D>(a, B, I);
  else
    gram_stage_strips<D, true>(a, B, I);
  __syncthreads();
  if (helper) tinv_offdiag(I, B);
  __syncthreads();
  // pieces 0..319 Tm, 320..639 P, then 48 pieces of factors (e^G, c e^G,
  // c e^{G_n - G}: contiguous from B.eg)
  const __amdgpu_buffer_rsrc_t r =
      rows_rsrc(a.sc + (((long long)b * a.H + h) * U + jc) * kScanSubBytes, kScanSubBytes);
  constexpr int NPIECE = kScanSubBytes / 16;
  for (int k = threadIdx.x; k < NPIECE; k += G::NT) {
    const hb* src = k < kTmPieces ? B.tt + tm_piece_lds(k)
                    : k < 2 * kTmPieces ? B.pp + tm_piece_lds(k - kTmPieces)
                                        : reinterpret_cast<const hb*>(B.eg + 4 * (k - 2 * kTmPieces));
    const uint4 x = *reinterpret_cast<const uint4*>(src);
    __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{x.x, x.y, x.z, x.w}, r, (uint32_t)(16 * k), 0, 0);
  }
}

template <int D>
struct ScanLay {
  static constexpr int DP = Geo<D>::DP;
  static constexpr int KR = (KRows<D>::ELEMS * 2 + 15) / 16 * 16;
  static constexpr int TT = CH * LDT * 2;
  static constexpr int LVT = CH + 4;   // fp32 stride of the transposed value strip
  static constexpr int o_kr = 0, o_qr = KR, o_tt = 2 * KR, o_pp = o_tt + TT, o_gf = o_pp + TT;
  static constexpr int o_vt = o_gf + 3 * CH * 4;
  static constexpr int BUF = o_vt + 16 * LVT * 4;   // one sub-chunk buffer (two alternate)
  static constexpr int LH = DP + 8;                 // fp16 stride of the transposed state strip
  static constexpr int LR = CH + 8;                 // fp16 stride of the transposed token strips
  static constexpr int HH = 16 * LH * 2;            // one copy of the state strip
  static constexpr int o_hh = 2 * BUF;              // two: read in one sub-chunk, written for the next
  static constexpr int BYTES = o_hh + 2 * HH;
  static constexpr int NC = 256;                              // compute threads: four wavefronts
  static constexpr int NS = 256;                              // stager threads: four wavefronts
  static constexpr int NKQ = (CH * (D / 8) + NS - 1) / NS;    // 16-byte K (and Q) pieces per stager thread
  static constexpr int NM = (2 * kTmPieces + NS - 1) / NS;    // Tm and P pieces per stager thread
  static_assert(BYTES <= 160 * 1024, "workgroup LDS budget exceeded");
  static_assert(BUF % 16 == 0 && KR % 16 == 0, "alignment");
};

// Rows of one sub-chunk of the strip scan in a stager thread's registers.
template <int D>
struct ScanStage {
  uint4 k[ScanLay<D>::NKQ], q[ScanLay<D>::NKQ], m[ScanLay<D>::NM], v, gf;
};

template <int D, bool OB>
__global__ __launch_bounds__(ScanLay<D>::NC + ScanLay<D>::NS) void sc_scan_kernel(Args a) {
  using G = Geo<D>;
  using SL = ScanLay<D>;
  constexpr int MD = G::MD, NP = G::NP, NC = SL::NC, NS = SL::NS;
  __shared__ __attribute__((aligned(16))) char smem[SL::BYTES];
  // XCD-aware mapping: workgroups are dealt to the 8 XCDs in turn, so
  // workgroup i = 8 j + x runs on XCD x; the strips of one head share an
  // XCD (and its L2, through which each of them reads all of the head's rows).
  const int x = (int)blockIdx.x & 7, j = (int)blockIdx.x >> 3;
  const int bh_ = x + 8 * (j / MD), s = j % MD;
  if (bh_ >= a.B * a.H) return;
  const int b = bh_ / a.H, h = bh_ % a.H;
  // waves 0-3 compute (wave r: row tile r of each sub-chunk), waves 4-7
  // stage the rows of the sub-chunks ahead (thread t of the stagers)
  const int r = wave_id(), lane = threadIdx.x & 63, g = lane >> 4, cl = lane & 15;
  const bool stager = r >= 4;
  const int t = (int)threadIdx.x - NC;
  const bool rev = a.dir == 1;
  const long long U = (a.T + CH - 1) / CH;
  const int HD = a.H * D;
  const long long hbase = ((long long)b * a.T) * HD + (long long)h * D;   // element of (b, token 0, h, 0)
  for (int i = threadIdx.x; i < SL::BYTES / 16; i += NC + NS) reinterpret_cast<uint4*>(smem)[i] = make_uint4(0, 0, 0, 0);
  auto sub = [&](long long jj) {   // sub-chunk jj in scan order (past the end: empty)
    const long long jc = rev ? U - 1 - jj : jj;
    const long long t0 = jj < U ? jc * CH : 0;
    return make_sub(t0, jj < U ? (int)(a.T - t0 < CH ? a.T - t0 : CH) : 0, rev);
  };
  auto fetch = [&](long long jj, ScanStage<D>& st) {
    const Sub sb = sub(jj);
    const __amdgpu_buffer_rsrc_t rk = rows_rsrc(a.k + hbase + sb.t0 * HD, (long long)sb.n * HD * 2);
    const __amdgpu_buffer_rsrc_t rq = rows_rsrc(a.q + hbase + sb.t0 * HD, (long long)sb.n * HD * 2);
#pragma unroll
    for (int i = 0; i < SL::NKQ; ++i) {   // pieces past the rows read past the buffer
      const int k = t + NS * i, row = k / (D / 8), c8 = k % (D / 8);
      const uint32_t off = (uint32_t)((sb.r0 + sb.sgn * row) * HD * 2 + 16 * c8);
      const u32x4_t vk = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
      const u32x4_t vq = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
      st.k[i] = make_uint4(vk[0], vk[1], vk[2], vk[3]);
      st.q[i] = make_uint4(vq[0], vq[1], vq[2], vq[3]);
    }
    const __amdgpu_buffer_rsrc_t rm = rows_rsrc(a.sc + (((long long)b * a.H + h) * U + sb.t0 / CH) * kScanSubBytes,
                                                sb.n > 0 ? kScanSubBytes : 0);
#pragma unroll
    for (int i = 0; i < SL::NM; ++i) {
      const u32x4_t vm = __builtin_amdgcn_raw_buffer_load_b128(rm, (uint32_t)(16 * (t + NS * i)), 0, 0);
      st.m[i] = make_uint4(vm[0], vm[1], vm[2], vm[3]);
    }
    // factors: pieces 640 .. 687 (threads 0..47; the others read past the end)
    const u32x4_t vg = __builtin_amdgcn_raw_buffer_load_b128(rm, (uint32_t)(16 * (2 * kTmPieces + (t < 48 ? t : 64))), 0, 0);
    st.gf = make_uint4(vg[0], vg[1], vg[2], vg[3]);
    // value strip: row t / 2, columns 16 s + 8 (t % 2) .. + 7 (threads 0..127)
    const __amdgpu_buffer_rsrc_t rv = rows_rsrc(a.v + hbase + sb.t0 * HD, (long long)sb.n * HD * 2);
    const int vrow = t >> 1;
    const u32x4_t vv = __builtin_amdgcn_raw_buffer_load_b128(
        rv, (uint32_t)(((sb.r0 + sb.sgn * vrow) * HD + 16 * s + 8 * (t & 1)) * 2), 0, 0);
    st.v = make_uint4(vv[0], vv[1], vv[2], vv[3]);
  };
  auto stage = [&](int buf, const ScanStage<D>& st) {
    char* p = smem + buf * SL::BUF;
    hb* kr = reinterpret_cast<hb*>(p + SL::o_kr);
    hb* qr = reinterpret_cast<hb*>(p + SL::o_qr);
#pragma unroll
    for (int i = 0; i < SL::NKQ; ++i) {
      const int k = t + NS * i, row = k / (D / 8), c8 = k % (D / 8);
      if (k < CH * (D / 8)) {
        *reinterpret_cast<uint4*>(kr + krow<D>(row) + 8 * c8) = bf16x8_to_f16x8(st.k[i]);
        *reinterpret_cast<uint4*>(qr + krow<D>(row) + 8 * c8) = bf16x8_to_f16x8(st.q[i]);
      }
    }
    hb* tt = reinterpret_cast<hb*>(p + SL::o_tt);
    hb* pp = reinterpret_cast<hb*>(p + SL::o_pp);
#pragma unroll
    for (int i = 0; i < SL::NM; ++i) {
      const int k = t + NS * i;
      if (k < kTmPieces)
        *reinterpret_cast<uint4*>(tt + tm_piece_lds(k)) = st.m[i];
      else if (k < 2 * kTmPieces)
        *reinterpret_cast<uint4*>(pp + tm_piece_lds(k - kTmPieces)) = st.m[i];
    }
    if (t < 48) *reinterpret_cast<uint4*>(p + SL::o_gf + 16 * t) = st.gf;
    if (t < 128) {
      float* vt = reinterpret_cast<float*>(p + SL::o_vt);
      const int row = t >> 1, c0 = 8 * (t & 1);
      const uint32_t w[4] = {st.v.x, st.v.y, st.v.z, st.v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vt[(c0 + 2 * e) * SL::LVT + row] = __uint_as_float(w[e] << 16);
        vt[(c0 + 2 * e + 1) * SL::LVT + row] = __uint_as_float(w[e] & 0xffff0000u);
      }
    }
  };
  // the state strip of sub-chunk jj (fp16, transposed): copy jj & 1
  auto hh = [&](long long jj) { return reinterpret_cast<hb*>(lds_at(smem, (uint32_t)(SL::o_hh + (jj & 1) * SL::HH))); };
  // state tiles of this wave: rows 16 md .. of the strip, md = r and r + 4
  constexpr int NMT = (MD + 3) / 4;
  f32x4 Hm[NMT];
  const size_t sbase = ((size_t)b * a.H + h) * D * D;
  const uint32_t so = (uint32_t)((4 * g * D + 16 * s + cl) * 4);   // lane byte offset within a state
  if (!stager) {
    const __amdgpu_buffer_rsrc_t hr = block_rsrc(a.h0 ? a.h0 + sbase : nullptr, a.h0 ? D * D * 4 : 0);
#pragma unroll
    for (int i = 0; i < NMT; ++i) {
      const int md = r + 4 * i;
#pragma unroll
      for (int e = 0; e < 4; ++e) Hm[i][e] = block_load(hr, so, (uint32_t)(((md < MD ? md : 0) * 16 + e) * D * 4));
    }
  }
  constexpr bool half = OB;
  const long long esz = half ? 2 : 4;
  // The two roles run their own loops with the same barriers (three per
  // sub-chunk), so that the compiler's waits before staging count only the
  // stagers' loads: with the register sets of two sub-chunks in flight, the
  // rows staged during sub-chunk jj were requested two sub-chunks earlier.
  // Both loops take an even number of steps (a last, empty one when U is odd:
  // its rows read as zeros, its stores fall outside the buffers, and it leaves
  // the state alone).
  if (stager) {
    ScanStage<D> s0, s1;   // rows of the even and the odd sub-chunks
    fetch(0, s0);
    __syncthreads();   // zero fill done
    stage(0, s0);
    fetch(1, s1);
    fetch(2, s0);
    __syncthreads();
    // during sub-chunk jj: stage jj + 1 into the other buffer (last read
    // before the end of jj - 1), then request jj + 3 into the same set
    auto sstep = [&](long long jj, ScanStage<D>& st) {
      stage((int)((jj + 1) & 1), st);
      fetch(jj + 3, st);
      __syncthreads();
    };
    for (long long jj = 0; jj < U; jj += 2) {
      sstep(jj, s1);
      sstep(jj + 1, s0);
    }
    return;
  }
  __syncthreads();   // zero fill done
#pragma unroll
  for (int i = 0; i < NMT; ++i) {
    const int md = r + 4 * i;
    if (md < MD) store4_h(hh(0) + cl * SL::LH + 16 * md + 4 * g, Hm[i][0], Hm[i][1], Hm[i][2], Hm[i][3]);
  }
  __syncthreads();
  auto cstep = [&](long long jj) {
    const Sub sb = sub(jj);
    const char* pc = smem + (jj & 1) * SL::BUF;
    const hb* kr = reinterpret_cast<const hb*>(pc + SL::o_kr);
    const hb* qr = reinterpret_cast<const hb*>(pc + SL::o_qr);
    const hb* tt = reinterpret_cast<const hb*>(pc + SL::o_tt);
    const hb* pp = reinterpret_cast<const hb*>(pc + SL::o_pp);
    const float* vt = reinterpret_cast<const float*>(pc + SL::o_vt);
    const float* eg = reinterpret_cast<const float*>(pc + SL::o_gf);
    const float* ce = eg + CH;
    const float* dn = eg + 2 * CH;
    // K H for all four row tiles (lane: rows 16 mt + 4 g .., column cl) and
    // (Q H)^T for this wave's tile (lane: token 16 r + cl, columns 4 g ..).
    // Every wave forms the whole R = V - c e^G K H and V' = Tm diag(beta) R
    // of the strip in registers (products repeated in the four waves), so
    // that a sub-chunk exchanges only the state strip: one barrier each.
    f32x4 qh = zero4(), kh[4];
    {
      const hb* hs = hh(jj);
      f16x8_t Hf[NP];
#pragma unroll
      for (int p = 0; p < NP; ++p)
        Hf[p] = cat8(ld4(hs + cl * SL::LH + 32 * p + 4 * g), ld4(hs + cl * SL::LH + 32 * p + 16 + 4 * g));
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) kh[mt] = zero4();
#pragma unroll
      for (int p = 0; p < NP; ++p) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) kh[mt] = mfma32(fragK<D>(kr + krow<D>(16 * mt + cl), p, g), Hf[p], kh[mt]);
        qh = mfma32(Hf[p], fragK<D>(qr + krow<D>(16 * r + cl), p, g), qh);
      }
    }
    // Lane holds R and V' rows 16 mt + 4 g .., column cl: tiles (0, 1) and
    // (2, 3) are the fp16 operand pairs of the token contractions below.
    f16x8_t Vh[2], Vs[2];
    {
      f32x4 R[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        R[mt] = ld4f(vt + cl * SL::LVT + 16 * mt + 4 * g) - ld4f(ce + 16 * mt + 4 * g) * kh[mt];
      const f16x8_t r0 = tof16x8(R[0], R[1]), r1 = tof16x8(R[2], R[3]);
      f32x4 vn[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        vn[mt] = mfma32(fragA2(tt + (16 * mt + cl) * LDT, 0, g), r0, zero4());
        if (mt >= 2) vn[mt] = mfma32(fragA2(tt + (16 * mt + cl) * LDT, 2, g), r1, vn[mt]);
      }
      Vh[0] = tof16x8(vn[0], vn[1]);
      Vh[1] = tof16x8(vn[2], vn[3]);
      f32x4 d4[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) d4[mt] = ld4f(dn + 16 * mt + 4 * g);
      Vs[0] = tof16x8(vn[0] * d4[0], vn[1] * d4[1]);
      Vs[1] = tof16x8(vn[2] * d4[2], vn[3] * d4[3]);
    }
    // outputs: O^T = e^G (Q H)^T + (P V')^T, lane: token 16 r + cl, columns 16 s + 4 g ..
    {
      f32x4 O = eg[16 * r + cl] * qh;
      O = mfma32(Vh[0], fragA2(pp + (16 * r + cl) * LDT, 0, g), O);
      if (r >= 2) O = mfma32(Vh[1], fragA2(pp + (16 * r + cl) * LDT, 2, g), O);
      const __amdgpu_buffer_rsrc_t ro =
          rows_rsrc(static_cast<char*>(a.out) + (hbase + sb.t0 * HD) * esz, (long long)sb.n * HD * esz);
      const uint32_t off = (uint32_t)(((sb.r0 + sb.sgn * (16 * r + cl)) * HD + 16 * s + 4 * g) * esz);
      if constexpr (half) {
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        const u32x2_t w{f32_to_bf16_bits(O[0]) | ((uint32_t)f32_to_bf16_bits(O[1]) << 16),
                        f32_to_bf16_bits(O[2]) | ((uint32_t)f32_to_bf16_bits(O[3]) << 16)};
        __builtin_amdgcn_raw_buffer_store_b64(w, ro, off, 0, 0);
      } else {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, O), ro, off, 0, 0);
      }
    }
    // state: H <- e^{G_n} H + K^T (c e^{G_n - G} V') for this wave's tiles
    if (jj < U) {
      const hb* kt = kr + krow<D>(4 * g + (cl >> 2)) + 4 * (cl & 3);
      const float dec = eg[CH - 1];
#pragma unroll
      for (int i = 0; i < NMT; ++i) {
        const int md = r + 4 * i;
        if (md < MD) {
          const f16x8_t k0 = cat8(ld4_tr(kt + 16 * md), ld4_tr(kt + krow<D>(16) + 16 * md));
          const f16x8_t k1 = cat8(ld4_tr(kt + krow<D>(32) + 16 * md), ld4_tr(kt + krow<D>(48) + 16 * md));
          f32x4 X = Hm[i] * dec;
          X = mfma32(k0, Vs[0], X);
          X = mfma32(k1, Vs[1], X);
          Hm[i] = X;
          store4_h(hh(jj + 1) + cl * SL::LH + 16 * md + 4 * g, X[0], X[1], X[2], X[3]);
        }
      }
    }
    __syncthreads();
  };
  for (long long jj = 0; jj < U; jj += 2) {
    cstep(jj);
    cstep(jj + 1);
  }
  if (a.hT) {
    const __amdgpu_buffer_rsrc_t hr = block_rsrc(a.hT + sbase, D * D * 4);
#pragma unroll
    for (int i = 0; i < NMT; ++i) {
      const int md = r + 4 * i;
      if (md < MD) {
#pragma unroll
        for (int e = 0; e < 4; ++e) block_store(hr, so, (uint32_t)((md * 16 + e) * D * 4), Hm[i][e]);
      }
    }
  }
}

struct Plan {
  int L, NS, ndir, dirs;
  bool cc;       // chunk-causal: forward maps and chain only; the reversed scan runs per chunk
  bool scan;     // strip scan (no maps, no chain): short single-direction calls
  ChainWs cw;    // split of the chain
  size_t maps_off, starts_off, acc_off, fac_off, gmaps_off, gstarts_off, tm_off, tm_bytes, bytes;
};

// Single-direction calls of at most this many 64-token sub-chunks per head
// take the strip scan.
constexpr long long kScanMaxSub = 32;
bool strip_scan(const Problem& p, int direction) {
  return (direction == GDN_FORWARD || direction == GDN_BACKWARD) && !p.prologue && p.strip_scan &&
         (p.T + CH - 1) / CH <= kScanMaxSub;
}

// Whether the output kernels of a two-scan call load the map kernels' Tm
// blocks instead of forming them.  At d_k <= 64 the helper wavefront's
// triangular inverse, the same work at every width, is the longest step of an
// output sub-chunk (the batched 2 x 35 x 64 workload, bidirectional: output
// launches 1.78 -> 1.36 ms, 6.43 -> 5.57 ms a step); at d_k = 112 the strips
// are, and loading measured no faster while moving 0.67 GB more per step
// through HBM.  The feature prologue's Q-only map kernel stores none (see
// seg_map_body).
bool tm_two_scan(const Problem& p) { return p.dk <= 64 && !p.prologue; }

Plan make_plan(const Problem& p, int direction) {
  Plan pl{};
  pl.cc = direction == GDN_CHUNK_CAUSAL;
  pl.dirs = direction == GDN_FORWARD || pl.cc ? 1 : direction == GDN_BACKWARD ? 2 : 3;
  pl.ndir = pl.dirs == 3 ? 2 : 1;
  if (strip_scan(p, direction)) {
    // one segment of the whole sequence; the workspace holds the prepared sub-chunks
    pl.scan = true;
    pl.NS = 1;
    pl.L = (int)((p.T + CH - 1) / CH * CH);
    pl.bytes = align_up((size_t)p.B * p.H * (size_t)((p.T + CH - 1) / CH) * kScanSubBytes, 256);
    return pl;
  }
  int L = p.segment_tokens;
  if (L <= 0) {
    // Segments per (batch, head).  Map and output workgroups run about one
    // per CU, and the grid's segment index is padded to a multiple of 8 with
    // workgroups dealt to the 8 XCDs (32 CUs each) in turn, so the busiest
    // XCD holds hb * ceil(ns / 8) of them: a launch takes about
    // ceil(hb * ceil(ns / 8) / 32) rounds of ceil(U / ns) + 1 sub-chunk steps
    // (one for a workgroup's start).  Take the count with the fewest such
    // steps, the smaller on ties, among 1..8 and multiples of 8 (whole rounds
    // of the XCDs).  Measured: the 60 s clip keeps 64 segments (2.07 ms a
    // bidirectional step, the best of lengths from 1408 to 2816 tokens); the
    // batched 2 x 35 x 64 workload 19 -> 40 segments, 5.60 -> 4.58 ms
    // (forward 2.90 -> 2.46 ms); the 5 s clip 33 -> 23 segments, 0.560 ->
    // 0.535 ms (forward 0.356 -> 0.305 ms).  Across 8 lengths of the batched
    // workload this count predicted the step time within 4%.
    const long long hb = (long long)p.B * p.H;
    const long long U = (p.T + CH - 1) / CH;
    // Short sequences: the chain's serial steps (one per segment, each about
    // as long as a sub-chunk step of the map and output kernels) would
    // outweigh the per-segment work, so keep at most about 2 sqrt(U)
    // segments for U sub-chunks (one 880-token frame: 7 segments of 128
    // tokens, 60 against 92 us a step with 14 segments of 64).
    long long cap = 1;
    while ((cap + 1) * (cap + 1) <= 4 * U) ++cap;
    long long want = 1, best = -1;
    for (long long ns = 1; ns <= cap; ns = ns < 8 ? ns + 1 : ns + 8) {
      const long long rounds = (hb * ((ns + 7) / 8) + 31) / 32;
      const long long steps = rounds * ((U + ns - 1) / ns + 1);
      if (best < 0 || steps < best) {
        best = steps;
        want = ns;
      }
    }
    long long per = (p.T + want - 1) / want;
    L = (int)((per + CH - 1) / CH * CH);
  }
  L = (L + CH - 1) / CH * CH;
  if (L < CH) L = CH;
  if ((long long)L > p.T) L = (int)((p.T + CH - 1) / CH * CH);
  pl.L = L;
  pl.NS = (int)((p.T + L - 1) / L);
  const size_t bhd = (size_t)pl.ndir * p.B * p.H;
  const size_t maps = bhd * (size_t)pl.NS * p.dk * (p.dk + p.dv) * sizeof(float);
  const size_t starts = bhd * (size_t)pl.NS * p.dk * p.dv * sizeof(float);
  // fp16 partial of the first output launch of a two-scan call
  const size_t acc = (pl.dirs == 3 || pl.cc) ? (size_t)p.B * p.T * p.H * p.dv * 2 : 0;
  pl.maps_off = 0;
  pl.starts_off = align_up(maps, 256);
  pl.acc_off = pl.starts_off + align_up(starts, 256);
  pl.fac_off = pl.acc_off + align_up(acc, 256);
  // bidirectional calls never split the chain (see launch_d)
  if (pl.dirs != 3) pl.cw = chain_ws(pl.NS - 1, p.chain_group, bhd, p.dk, p.dv);
  pl.gmaps_off = pl.fac_off + align_up(prologue_bytes(p), 256);
  pl.gstarts_off = pl.gmaps_off + pl.cw.gmaps_bytes;
  // Tm blocks of every sub-chunk of each scan with maps (fp16, 5 KB per
  // sub-chunk and head), whether or not the output kernels load them: the
  // scan of a forward- or backward-only call, and for d_k <= 64 (without
  // the feature prologue) both scans of a bidirectional call and the forward
  // scan of a chunk-causal one (see launch_d)
  const size_t U = (size_t)((p.T + CH - 1) / CH);
  const bool two_scan = pl.dirs == 3 || pl.cc;
  const size_t tm_slots = pl.NS < 2 ? 0 : !two_scan ? 1 : !tm_two_scan(p) ? 0 : pl.cc ? 1 : 2;
  pl.tm_bytes = tm_slots ? align_up(tm_slots * p.B * p.H * U * kTmElems * 2, 256) : 0;
  pl.tm_off = pl.gstarts_off + pl.cw.gstarts_bytes;
  pl.bytes = pl.tm_off + pl.tm_bytes;
  return pl;
}

// The chain of `nsl` scan slots from a.slot0, whole or split (compose, chain
// of groups, expand); `pt`: the reversed scan of a bidirectional call.
template <int D>
hipError_t chain_launch(Args a, const ChainWs& cw, unsigned bhc, unsigned nsl, bool pt, hipStream_t st,
                        bool split = true) {
  a.ch_m = cw.m;
  a.ch_groups = cw.groups;
  if (!split) a.ch_m = a.ch_groups = 0;
  auto go = [&](int mode, unsigned gz, bool ptv) -> hipError_t {
    a.ch_mode = mode;
    if (mode == 0 || mode == 2) {   // serial chains: two column-group workgroups per head
      using SC = ChainSplitCols<D, true>;
      const dim3 grid(bhc, nsl * SC::NH, gz), block(64 * SC::NW);
      if (ptv)
        hipLaunchKernelGGL((seg_chain_kernel<D, true, true>), grid, block, 0, st, a);
      else
        hipLaunchKernelGGL((seg_chain_kernel<D, false, true>), grid, block, 0, st, a);
    } else {
      using SC = ChainSplitCols<D, false>;
      const dim3 grid(bhc, nsl * SC::NH, gz), block(64 * SC::NW);
      if (ptv)
        hipLaunchKernelGGL((seg_chain_kernel<D, true, false>), grid, block, 0, st, a);
      else
        hipLaunchKernelGGL((seg_chain_kernel<D, false, false>), grid, block, 0, st, a);
    }
    return hipGetLastError();
  };
  if (a.ch_m == 0) return go(0, 1, pt);
  hipError_t e;
  if ((e = go(1, 2 * cw.groups, pt)) != hipSuccess) return e;
  if ((e = go(2, 1, false)) != hipSuccess) return e;
  return go(3, cw.groups, pt);
}

// Library-owned side streams (default priority) with a fork and a join event,
// for the concurrent part of two-scan calls: per device, one for each of up
// to kSides caller streams, bound on first use and kept until the process
// ends.  A call whose stream finds no free entry (or whose side stream cannot
// be created) runs in order on its own stream.  The entry's mutex makes a
// call's fork, launches and join one unit with respect to calls on the same
// caller stream from other host threads; calls on different streams do not
// wait for each other.
struct Side {
  std::mutex mu;
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};

Side* side_stream(hipStream_t caller) {
  constexpr int kMaxDevices = 64, kSides = 8;
  struct Dev {
    std::mutex mu;                 // guards the binding of entries to caller streams
    int used = 0;
    hipStream_t owner[kSides] = {};
    Side side[kSides];
  };
  static Dev devs[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  Dev& d = devs[dev];
  std::lock_guard<std::mutex> lk(d.mu);
  for (int i = 0; i < d.used; ++i)
    if (d.owner[i] == caller) return d.side[i].stream ? &d.side[i] : nullptr;
  if (d.used == kSides) return nullptr;
  Side& s = d.side[d.used];
  d.owner[d.used++] = caller;
  if (hipStreamCreateWithFlags(&s.stream, hipStreamNonBlocking) != hipSuccess ||
      hipEventCreateWithFlags(&s.fork, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&s.join, hipEventDisableTiming) != hipSuccess) {
    s.stream = nullptr;   // this caller stream runs in order from now on
    return nullptr;
  }
  return &s;
}

template <int D, bool PRO>
hipError_t launch_d(const Problem& p, const Plan& pl, const Tensors& t, char* ws, hipStream_t stream) {
  Args a{};
  if constexpr (PRO) {
    // the factors first, on the call's stream (every later launch, and the
    // side stream's fork, is ordered after it)
    float* fac = reinterpret_cast<float*>(ws + pl.fac_off);
    const hipError_t e = prologue_launch(p, t, fac, stream);
    if (e != hipSuccess) return e;
    a.fac = fac;
  }
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
  a.part = reinterpret_cast<hb*>(ws + pl.acc_off);
  a.T = p.T;
  a.B = p.B;
  a.H = p.H;
  a.L = pl.L;
  a.NS = pl.NS;
  a.dirs = pl.dirs;
  a.out_bf16 = p.out_bf16 ? 1 : 0;
  a.c = p.key_scale;
  a.gmaps = reinterpret_cast<float*>(ws + pl.gmaps_off);
  a.gstarts = reinterpret_cast<float*>(ws + pl.gstarts_off);
  if constexpr (!PRO) {
    if (pl.scan) {
      a.sc = ws;
      a.dir = pl.dirs == 1 ? 0 : 1;
      const unsigned U = (unsigned)((p.T + CH - 1) / CH), nbh = (unsigned)(p.B * p.H);
      prof_begin(stream, GDN_KERNEL_SCAN_PREP);
      hipLaunchKernelGGL((sc_prep_kernel<D>), dim3(U, nbh, 1), dim3(Geo<D>::NT), 0, stream, a);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      prof_end(stream, GDN_KERNEL_SCAN_PREP);
      // 8 x (strips x ceil(heads / 8)) workgroups: the strips of a head on one XCD
      const unsigned gx = 8u * (unsigned)Geo<D>::MD * ((nbh + 7u) / 8u);
      prof_begin(stream, GDN_KERNEL_SCAN);
      if (p.out_bf16)
        hipLaunchKernelGGL((sc_scan_kernel<D, true>), dim3(gx, 1, 1), dim3(ScanLay<D>::NC + ScanLay<D>::NS), 0, stream, a);
      else
        hipLaunchKernelGGL((sc_scan_kernel<D, false>), dim3(gx, 1, 1), dim3(ScanLay<D>::NC + ScanLay<D>::NS), 0, stream, a);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      prof_end(stream, GDN_KERNEL_SCAN);
      return hipSuccess;
    }
  }
  const bool both = pl.dirs == 3;
  // Reuse of the map kernel's Tm blocks by the output kernel: forward- and
  // backward-only calls (measured at the 60 s clip, output kernel alone:
  // 0.613 -> 0.590 ms for a forward call), and two-scan calls at d_k <= 64
  // (see tm_two_scan).
  a.tm = pl.tm_bytes && p.tm_reuse ? reinterpret_cast<hb*>(ws + pl.tm_off) : nullptr;
  const unsigned bhc = (unsigned)(p.B * p.H);
  // Workgroups are dealt to the 8 XCDs (each with its own L2) in turn.  With
  // the segment index padded to a multiple of 8, a segment of neighbouring
  // heads lands on the same XCD, so the cache lines their rows share (a head's
  // slice of a token row is not line-aligned) are fetched from memory once.
  auto padded = [](int n) { return (unsigned)((n + 7) / 8 * 8); };
  // Maps of the scan in `slot`: segments 0 .. NS-2 in scan order, and also the
  // last one for the forward scan of a bidirectional call (its transpose is
  // the reversed scan's first P) and wherever the output kernels reuse the
  // map kernels' Tm blocks; the reversed scan of a bidirectional call forms Q
  // only.
  // In a bidirectional call the second map and output launches visit the heads
  // in reversed order, so that they start on the heads whose inputs (and
  // partial outputs) the first launch touched last, which the memory-side
  // cache may still hold.
  auto maps_k = [&](int slot, hipStream_t st) -> hipError_t {
    if (pl.NS < 2) return hipSuccess;
    a.slot0 = slot;
    a.heads_rev = both && slot == 1;
    prof_begin(st, GDN_KERNEL_SEG_MAP);
    a.npos = (both && slot == 0) || a.tm ? pl.NS : pl.NS - 1;
    if (both && slot == 1)
      hipLaunchKernelGGL((seg_map_q_kernel<D, PRO>), dim3(padded(a.npos), bhc, 1), dim3(Geo<D>::NT), 0, st, a);
    else
      hipLaunchKernelGGL((seg_map_kernel<D, PRO>), dim3(padded(a.npos), bhc, 1), dim3(Geo<D>::NT), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    prof_end(st, GDN_KERNEL_SEG_MAP);
    return hipSuccess;
  };
  // Chain of the scan in `slot`.
  // The split chain (many workgroups for a short time) pays off where the
  // chain stands alone on the critical path; beside the other scan's maps
  // and outputs in the two-stream bidirectional schedule, the single
  // workgroup pair per head is faster (measured at the 60 s clip: splitting
  // both chains 2.46 against 2.33 ms per step, splitting the forward chain
  // alone 2.32 against 2.10 ms), so bidirectional calls never split (in
  // either schedule, which keeps the two schedules' results identical).
  auto chain_k = [&](int slot, hipStream_t st) -> hipError_t {
    a.slot0 = slot;
    prof_begin(st, GDN_KERNEL_SEG_CHAIN);
    const hipError_t e = chain_launch<D>(a, pl.cw, bhc, 1, both && slot == 1, st, !both);
    if (e != hipSuccess) return e;
    prof_end(st, GDN_KERNEL_SEG_CHAIN);
    return hipSuccess;
  };
  // One output launch (x.mode and x.out_bf16 select the store type).
  // x.tm: load the map kernel's Tm blocks.
  // (Loaded Tm blocks occur in single-scan calls, mode 0, and in two-scan
  // calls only where tm_two_scan allows: the partial-storing and -adding
  // variants with loaded blocks are built for d_k <= 64 without the prologue.)
  auto launch_out = [&](const Args& x, unsigned gx, hipStream_t st) {
    const dim3 grid(gx, bhc, 1), block(Geo<D>::NT);
    if (x.tm && x.mode == 0) {
      if (x.out_bf16)
        hipLaunchKernelGGL((seg_out_kernel<D, PRO, 1, true>), grid, block, 0, st, x);
      else
        hipLaunchKernelGGL((seg_out_kernel<D, PRO, 0, true>), grid, block, 0, st, x);
    } else if (x.tm) {
      if constexpr (D <= 64 && !PRO) {
        if (x.mode == 1)
          hipLaunchKernelGGL((seg_out_kernel<D, PRO, 2, true>), grid, block, 0, st, x);
        else if (x.out_bf16)
          hipLaunchKernelGGL((seg_out_kernel<D, PRO, 4, true>), grid, block, 0, st, x);
        else
          hipLaunchKernelGGL((seg_out_kernel<D, PRO, 3, true>), grid, block, 0, st, x);
      }
    } else if (x.mode == 1) {
      hipLaunchKernelGGL((seg_out_kernel<D, PRO, 2, false>), grid, block, 0, st, x);
    } else if (x.mode == 2) {
      if (x.out_bf16)
        hipLaunchKernelGGL((seg_out_kernel<D, PRO, 4, false>), grid, block, 0, st, x);
      else
        hipLaunchKernelGGL((seg_out_kernel<D, PRO, 3, false>), grid, block, 0, st, x);
    } else {
      if (x.out_bf16)
        hipLaunchKernelGGL((seg_out_kernel<D, PRO, 1, false>), grid, block, 0, st, x);
      else
        hipLaunchKernelGGL((seg_out_kernel<D, PRO, 0, false>), grid, block, 0, st, x);
    }
  };
  // Outputs of one scan direction; in a bidirectional call the forward scan
  // stores its partial and the reversed scan adds it.
  auto outputs = [&](int dir, hipStream_t st) -> hipError_t {
    a.dir = dir;
    a.mode = both ? (dir == 0 ? 1 : 2) : 0;
    a.heads_rev = both && dir == 1;
    prof_begin(st, GDN_KERNEL_SEG_OUT);
    a.npos = pl.NS;
    launch_out(a, padded(pl.NS), st);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    prof_end(st, GDN_KERNEL_SEG_OUT);
    return hipSuccess;
  };
  hipError_t e = hipSuccess;
  if (pl.cc) {
    // Chunk-causal: the reversed scan needs no maps or chain (each chunk
    // starts from zero), so it runs first, on the side stream, storing the
    // partial, beside the forward maps and chain; the forward outputs add it.
    const long long cf = (long long)p.first_chunk_frames * p.S, cl_ = (long long)p.chunk_frames * p.S;
    const int nchunks = p.T <= cf ? 1 : 1 + (int)((p.T - cf + cl_ - 1) / cl_);
    auto rev_chunks = [&](hipStream_t st) -> hipError_t {
      Args r = a;
      r.tm = nullptr;   // the chunks have no maps
      r.dir = 1;
      r.mode = 1;
      r.cs_first = cf;
      r.cs_len = cl_;
      r.npos = nchunks;
      prof_begin(st, GDN_KERNEL_SEG_OUT);
      launch_out(r, padded(nchunks), st);
      const hipError_t e2 = hipGetLastError();
      if (e2 != hipSuccess) return e2;
      prof_end(st, GDN_KERNEL_SEG_OUT);
      return hipSuccess;
    };
    auto fwd_out = [&](hipStream_t st) -> hipError_t {
      a.dir = 0;
      a.mode = 2;
      a.heads_rev = 0;
      a.npos = pl.NS;
      prof_begin(st, GDN_KERNEL_SEG_OUT);
      launch_out(a, padded(pl.NS), st);
      const hipError_t e2 = hipGetLastError();
      if (e2 != hipSuccess) return e2;
      prof_end(st, GDN_KERNEL_SEG_OUT);
      return hipSuccess;
    };
    Side* side = p.serial_scans ? nullptr : side_stream(stream);
    if (!side) {
      if ((e = rev_chunks(stream)) != hipSuccess) return e;
      if ((e = maps_k(0, stream)) != hipSuccess) return e;
      if ((e = chain_k(0, stream)) != hipSuccess) return e;
      return fwd_out(stream);
    }
    std::lock_guard<std::mutex> lk(side->mu);
    if ((e = hipEventRecord(side->fork, stream)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(side->stream, side->fork, 0)) != hipSuccess) return e;
    if ((e = rev_chunks(side->stream)) != hipSuccess) return e;
    if ((e = hipEventRecord(side->join, side->stream)) != hipSuccess) return e;
    if ((e = maps_k(0, stream)) != hipSuccess) return e;
    if ((e = chain_k(0, stream)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(stream, side->join, 0)) != hipSuccess) return e;
    return fwd_out(stream);
  }
  if (!both) {
    if ((e = maps_k(0, stream)) != hipSuccess) return e;
    if ((e = chain_k(0, stream)) != hipSuccess) return e;
    return outputs(pl.dirs == 1 ? 0 : 1, stream);
  }
  Side* side = p.serial_scans ? nullptr : side_stream(stream);
  if (!side) {
    if ((e = maps_k(0, stream)) != hipSuccess) return e;
    if ((e = maps_k(1, stream)) != hipSuccess) return e;
    if ((e = chain_k(0, stream)) != hipSuccess) return e;
    if ((e = chain_k(1, stream)) != hipSuccess) return e;
    if ((e = outputs(0, stream)) != hipSuccess) return e;
    return outputs(1, stream);
  }
  // Both scans, partly concurrent.  The serial chain kernels occupy two CUs
  // per head, so each runs beside a full-width kernel: the forward maps first
  // (alone; the reversed chain needs them too), then on the side stream the
  // reversed maps and chain beside the forward chain and outputs.  The
  // reversed outputs add the forward partial and so wait for both.  (Forward
  // maps and chain split into two pipelined halves, the first chain half
  // beside the second map half, measured slower: 2.20 against 2.14 ms per
  // step at the 60 s clip, as the reversed maps then start later.)
  std::lock_guard<std::mutex> lk(side->mu);
  if ((e = maps_k(0, stream)) != hipSuccess) return e;
  if ((e = hipEventRecord(side->fork, stream)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(side->stream, side->fork, 0)) != hipSuccess) return e;
  if ((e = maps_k(1, side->stream)) != hipSuccess) return e;
  if ((e = chain_k(1, side->stream)) != hipSuccess) return e;
  if ((e = hipEventRecord(side->join, side->stream)) != hipSuccess) return e;
  if ((e = chain_k(0, stream)) != hipSuccess) return e;
  if ((e = outputs(0, stream)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(stream, side->join, 0)) != hipSuccess) return e;
  return outputs(1, stream);
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
    case 16: return p.prologue ? launch_d<16, true>(p, pl, t, ws, stream) : launch_d<16, false>(p, pl, t, ws, stream);
    case 32: return p.prologue ? launch_d<32, true>(p, pl, t, ws, stream) : launch_d<32, false>(p, pl, t, ws, stream);
    case 48: return p.prologue ? launch_d<48, true>(p, pl, t, ws, stream) : launch_d<48, false>(p, pl, t, ws, stream);
    case 64: return p.prologue ? launch_d<64, true>(p, pl, t, ws, stream) : launch_d<64, false>(p, pl, t, ws, stream);
    case 80: return p.prologue ? launch_d<80, true>(p, pl, t, ws, stream) : launch_d<80, false>(p, pl, t, ws, stream);
    case 96: return p.prologue ? launch_d<96, true>(p, pl, t, ws, stream) : launch_d<96, false>(p, pl, t, ws, stream);
    case 112: return p.prologue ? launch_d<112, true>(p, pl, t, ws, stream) : launch_d<112, false>(p, pl, t, ws, stream);
    default: return hipErrorInvalidValue;
  }
}

int chunked_segment_tokens(const Problem& p, int direction) { return make_plan(p, direction).L; }

// --- frame-level (Jacobi) path ----------------------------------------------
namespace {
struct JacPlan {
  int ndir, dirs;
  ChainWs cw;
  size_t maps_off, starts_off, fac_off, gmaps_off, gstarts_off, bytes;
};
JacPlan jac_plan(const Problem& p, int direction) {
  JacPlan pl{};
  pl.dirs = direction == GDN_FORWARD ? 1 : direction == GDN_BACKWARD ? 2 : 3;
  pl.ndir = pl.dirs == 3 ? 2 : 1;
  const size_t per = (size_t)pl.ndir * p.B * p.H * (size_t)(p.F + 1);
  pl.maps_off = 0;
  pl.starts_off = align_up(per * p.dk * (p.dk + p.dv) * sizeof(float), 256);
  pl.fac_off = pl.starts_off + align_up(per * p.dk * p.dv * sizeof(float), 256);
  pl.cw = chain_ws(p.F, p.chain_group, (size_t)pl.ndir * p.B * p.H, p.dk, p.dv);
  pl.gmaps_off = pl.fac_off + align_up(prologue_bytes(p), 256);
  pl.gstarts_off = pl.gmaps_off + pl.cw.gmaps_bytes;
  pl.bytes = pl.gstarts_off + pl.cw.gstarts_bytes;
  return pl;
}

template <int D, bool PRO>
hipError_t jac_launch_d(const Problem& p, const JacPlan& pl, const Tensors& t, char* ws, hipStream_t stream) {
  Args a{};
  if constexpr (PRO) {
    float* fac = reinterpret_cast<float*>(ws + pl.fac_off);
    const hipError_t e = prologue_launch(p, t, fac, stream);
    if (e != hipSuccess) return e;
    a.fac = fac;
  }
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
  a.T = p.T;
  a.B = p.B;
  a.H = p.H;
  a.L = p.S;          // one frame per "segment"
  a.NS = p.F + 1;     // chain positions: the start of every frame and the end state
  a.dirs = pl.dirs;
  a.out_bf16 = p.out_bf16 ? 1 : 0;
  a.c = p.key_scale;
  const unsigned bhc = (unsigned)(p.B * p.H);
  hipError_t e;
  prof_begin(stream, GDN_KERNEL_JAC_MAP);
  hipLaunchKernelGGL((jac_map_kernel<D, PRO>), dim3(p.F, bhc), dim3(64 * (D / 16)), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  prof_end(stream, GDN_KERNEL_JAC_MAP);
  a.slot0 = 0;
  a.gmaps = reinterpret_cast<float*>(ws + pl.gmaps_off);
  a.gstarts = reinterpret_cast<float*>(ws + pl.gstarts_off);
  prof_begin(stream, GDN_KERNEL_SEG_CHAIN);
  if ((e = chain_launch<D>(a, pl.cw, bhc, (unsigned)pl.ndir, false, stream)) != hipSuccess) return e;
  prof_end(stream, GDN_KERNEL_SEG_CHAIN);
  prof_begin(stream, GDN_KERNEL_JAC_OUT);
  if (p.out_bf16)
    hipLaunchKernelGGL((jac_out_kernel<D, PRO, true>), dim3(p.F, bhc), dim3(64 * (D / 16)), 0, stream, a);
  else
    hipLaunchKernelGGL((jac_out_kernel<D, PRO, false>), dim3(p.F, bhc), dim3(64 * (D / 16)), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  prof_end(stream, GDN_KERNEL_JAC_OUT);
  return hipSuccess;
}
}  // namespace

const char* jacobi_unsupported_reason(const Problem& p) {
  if (!p.qkv_bf16) return "q, k and v must be bf16";
  if (p.dk != p.dv) return "d_k must equal d_v";
  if (p.dk > 112) return "d_k = d_v must be at most 112";
  if (p.B * (long long)p.H > 65535) return "batch * heads must be at most 65535";
  return nullptr;
}

size_t jacobi_workspace(const Problem& p, int direction) { return jac_plan(p, direction).bytes; }

hipError_t jacobi_launch(const Problem& p, int direction, const Tensors& t, void* workspace, hipStream_t stream) {
  const JacPlan pl = jac_plan(p, direction);
  char* ws = static_cast<char*>(workspace);
  switch (p.dk) {
    case 16: return p.prologue ? jac_launch_d<16, true>(p, pl, t, ws, stream) : jac_launch_d<16, false>(p, pl, t, ws, stream);
    case 32: return p.prologue ? jac_launch_d<32, true>(p, pl, t, ws, stream) : jac_launch_d<32, false>(p, pl, t, ws, stream);
    case 48: return p.prologue ? jac_launch_d<48, true>(p, pl, t, ws, stream) : jac_launch_d<48, false>(p, pl, t, ws, stream);
    case 64: return p.prologue ? jac_launch_d<64, true>(p, pl, t, ws, stream) : jac_launch_d<64, false>(p, pl, t, ws, stream);
    case 80: return p.prologue ? jac_launch_d<80, true>(p, pl, t, ws, stream) : jac_launch_d<80, false>(p, pl, t, ws, stream);
    case 96: return p.prologue ? jac_launch_d<96, true>(p, pl, t, ws, stream) : jac_launch_d<96, false>(p, pl, t, ws, stream);
    case 112: return p.prologue ? jac_launch_d<112, true>(p, pl, t, ws, stream) : jac_launch_d<112, false>(p, pl, t, ws, stream);
    default: return hipErrorInvalidValue;
  }
}


}  // namespace gdn
