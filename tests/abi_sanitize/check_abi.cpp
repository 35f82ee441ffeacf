// Host-only check of libgdn's C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer: every call below fails, sizes or plans on the
// host, before any HIP call (no GPU needed).  Built and run by
// tests/test_abi_sanitize.py; exits non-zero on the first mismatch.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "gdn.h"

static int failures = 0;
#define EXPECT(cond)                                                            \
  do {                                                                          \
    if (!(cond)) {                                                              \
      std::fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond);    \
      ++failures;                                                               \
    }                                                                           \
  } while (0)

static gdn_problem base() {
  gdn_problem p;
  std::memset(&p, 0, sizeof p);
  p.abi_version = GDN_ABI_VERSION;
  p.batch = 1;
  p.heads = 2;
  p.d_k = 64;
  p.d_v = 64;
  p.frames = 3;
  p.tokens_per_frame = 100;
  p.qkv_dtype = GDN_BF16;
  p.out_dtype = GDN_F32;
  p.algo = GDN_ALGO_AUTO;
  p.key_scale = 1.0f;
  return p;
}

// Deterministic 64-bit LCG for the field fuzz.
static uint64_t rng = 0x9e3779b97f4a7c15ull;
static int64_t draw(int64_t lo, int64_t hi) {
  rng = rng * 6364136223846793005ull + 1442695040888963407ull;
  return lo + (int64_t)((rng >> 33) % (uint64_t)(hi - lo + 1));
}

int main() {
  void* const fake = reinterpret_cast<void*>(uintptr_t{0x10000});
  size_t n = 0;
  int32_t tok = 0;
  // status text and version
  EXPECT(gdn_abi_version() == GDN_ABI_VERSION);
  for (int s = -1; s <= 5; ++s) EXPECT(gdn_status_string(s) != nullptr);
  EXPECT(std::strcmp(gdn_status_string(GDN_ERR_HIP), "GDN_ERR_HIP") == 0);
  // null and malformed problems
  EXPECT(gdn_workspace_size(nullptr, GDN_FORWARD, &n) == GDN_ERR_INVALID_ARGUMENT);
  EXPECT(std::strlen(gdn_last_error_message()) > 0);
  gdn_problem p = base();
  EXPECT(gdn_workspace_size(&p, GDN_FORWARD, nullptr) == GDN_ERR_INVALID_ARGUMENT);
  EXPECT(gdn_plan_segment_tokens(&p, GDN_FORWARD, nullptr) == GDN_ERR_INVALID_ARGUMENT);
  EXPECT(gdn_workspace_size(&p, 9, &n) == GDN_ERR_INVALID_ARGUMENT);
  struct Bad { int32_t gdn_problem::*f; int32_t v; };
  const Bad bad[] = {{&gdn_problem::abi_version, 1}, {&gdn_problem::batch, 0}, {&gdn_problem::heads, -3},
                     {&gdn_problem::d_k, 8}, {&gdn_problem::d_v, 144}, {&gdn_problem::frames, 0},
                     {&gdn_problem::tokens_per_frame, -1}, {&gdn_problem::qkv_dtype, 5},
                     {&gdn_problem::out_dtype, -2}, {&gdn_problem::algo, 7}, {&gdn_problem::intra, 3},
                     {&gdn_problem::prologue, 9}, {&gdn_problem::segment_tokens, -64},
                     {&gdn_problem::chain_group, -1}, {&gdn_problem::flags, 64}, {&gdn_problem::flags, 8}};
  for (const Bad& b : bad) {
    gdn_problem q = base();
    q.*(b.f) = b.v;
    EXPECT(gdn_workspace_size(&q, GDN_BIDIRECTIONAL, &n) == GDN_ERR_INVALID_ARGUMENT);
  }
  for (int i = 0; i < 5; ++i) {
    gdn_problem q = base();
    q.reserved[i] = 1;
    EXPECT(gdn_workspace_size(&q, GDN_FORWARD, &n) == GDN_ERR_INVALID_ARGUMENT);
  }
  {
    gdn_problem q = base();
    q.key_scale = std::nanf("");
    EXPECT(gdn_workspace_size(&q, GDN_FORWARD, &n) == GDN_ERR_INVALID_ARGUMENT);
    q = base();
    q.frames = 1 << 20;
    q.tokens_per_frame = 1 << 20;   // 2^40 tokens
    EXPECT(gdn_workspace_size(&q, GDN_FORWARD, &n) == GDN_ERR_INVALID_ARGUMENT);
  }
  // forward / step: nulls, misalignment, workspace too small, all before any HIP call
  p = base();
  p.algo = GDN_ALGO_RECURRENT;
  EXPECT(gdn_forward(&p, GDN_BIDIRECTIONAL, nullptr, fake, fake, (float*)fake, (float*)fake, nullptr, fake,
                     nullptr, nullptr, 0, nullptr) == GDN_ERR_INVALID_ARGUMENT);
  EXPECT(gdn_forward(&p, GDN_BIDIRECTIONAL, (char*)fake + 2, fake, fake, (float*)fake, (float*)fake, nullptr,
                     fake, nullptr, nullptr, 0, nullptr) == GDN_ERR_INVALID_ARGUMENT);
  EXPECT(gdn_forward(&p, GDN_BIDIRECTIONAL, fake, fake, fake, (float*)fake, (float*)fake, nullptr, fake, nullptr,
                     nullptr, 0, nullptr) == GDN_ERR_WORKSPACE_TOO_SMALL);
  p.frames = 2;
  EXPECT(gdn_step(&p, fake, fake, fake, (float*)fake, (float*)fake, nullptr, (float*)fake, fake, nullptr, 0,
                  nullptr) == GDN_ERR_INVALID_ARGUMENT);
  EXPECT(gdn_step_noalloc(&p, fake, fake, fake, (float*)fake, (float*)fake, nullptr, (float*)fake, fake,
                          nullptr) == GDN_ERR_INVALID_ARGUMENT);
  p = base();
  p.frames = 1;
  p.batch = 8;
  p.heads = 64;
  p.d_k = p.d_v = 112;
  p.tokens_per_frame = 60000;
  p.algo = GDN_ALGO_CHUNKED;
  EXPECT(gdn_step_noalloc(&p, fake, fake, fake, (float*)fake, (float*)fake, nullptr, (float*)fake, fake,
                          nullptr) == GDN_ERR_WORKSPACE_TOO_SMALL);
  // unsupported requests
  p = base();
  p.intra = GDN_INTRA_JACOBI;
  p.qkv_dtype = GDN_F32;
  EXPECT(gdn_workspace_size(&p, GDN_FORWARD, &n) == GDN_ERR_UNSUPPORTED);
  p = base();
  p.intra = GDN_INTRA_JACOBI;
  p.first_chunk_frames = p.chunk_frames = 1;
  EXPECT(gdn_workspace_size(&p, GDN_CHUNK_CAUSAL, &n) == GDN_ERR_UNSUPPORTED);
  // field fuzz: every combination either sizes (and plans) or is rejected, on
  // the host, with no sanitizer report; the sizes are monotone in the frames
  for (int it = 0; it < 20000; ++it) {
    gdn_problem q = base();
    q.batch = (int32_t)draw(-1, 70);
    q.heads = (int32_t)draw(-1, 70);
    q.d_k = (int32_t)(16 * draw(0, 9));
    q.d_v = (int32_t)(16 * draw(0, 9));
    q.frames = (int32_t)draw(0, 3000);
    q.tokens_per_frame = (int32_t)draw(0, 5000);
    q.qkv_dtype = (int32_t)draw(0, 1);
    q.out_dtype = (int32_t)draw(0, 1);
    q.algo = (int32_t)draw(0, 2);
    q.intra = (int32_t)draw(0, 1);
    q.prologue = (int32_t)draw(0, 1);
    q.first_chunk_frames = (int32_t)draw(0, 5);
    q.chunk_frames = (int32_t)draw(0, 5);
    q.segment_tokens = (int32_t)(draw(0, 3) == 0 ? draw(0, 1 << 20) : 0);
    q.chain_group = (int32_t)draw(0, 40);
    q.flags = (int32_t)draw(0, 7);
    const int32_t dir = (int32_t)draw(0, 3);
    const gdn_status s = gdn_workspace_size(&q, dir, &n);
    EXPECT(s == GDN_OK || s == GDN_ERR_INVALID_ARGUMENT || s == GDN_ERR_UNSUPPORTED);
    if (s == GDN_OK) {
      EXPECT(gdn_plan_segment_tokens(&q, dir, &tok) == GDN_OK);
      EXPECT(tok >= 0 && tok % 64 == 0);
      gdn_problem r = q;
      r.frames = q.frames + 1;
      size_t m = 0;
      if (gdn_workspace_size(&r, dir, &m) == GDN_OK && r.segment_tokens > 0) EXPECT(m >= n);
    } else {
      EXPECT(std::strlen(gdn_last_error_message()) > 0);
    }
  }
  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("abi host checks passed\n");
  return 0;
}
