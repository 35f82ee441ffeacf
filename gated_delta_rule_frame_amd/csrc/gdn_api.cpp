// C-ABI entry points of libgdn: argument validation, workspace sizing and
// dispatch to the kernel launchers.  Everything here runs on the host; no HIP
// call is made before every argument has been checked.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "gdn_internal.h"

namespace {

thread_local std::string g_last_error;

gdn_status fail(gdn_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks the problem descriptor and fills `out`.  `direction` < 0 skips the
// direction check (gdn_step).
gdn_status check_problem(const gdn_problem* pr, int direction, gdn::Problem* out) {
  if (!pr) return fail(GDN_ERR_INVALID_ARGUMENT, "problem is NULL");
  if (pr->abi_version != GDN_ABI_VERSION)
    return fail(GDN_ERR_INVALID_ARGUMENT, "abi_version %d != %d", pr->abi_version, GDN_ABI_VERSION);
  for (int i = 0; i < (int)(sizeof pr->reserved / sizeof pr->reserved[0]); ++i)
    if (pr->reserved[i] != 0) return fail(GDN_ERR_INVALID_ARGUMENT, "reserved[%d] is not zero", i);
  if (pr->flags & ~(GDN_FLAG_SERIAL_SCANS | GDN_FLAG_FORM_INVERSE | GDN_FLAG_NO_STRIP_SCAN))
    return fail(GDN_ERR_INVALID_ARGUMENT, "unknown flags 0x%x", (unsigned)pr->flags);
  if (pr->segment_tokens < 0 || pr->segment_tokens > (1 << 30))
    return fail(GDN_ERR_INVALID_ARGUMENT, "segment_tokens must be in [0, 2^30] (got %d)", pr->segment_tokens);
  if (pr->chain_group < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "chain_group must be >= 0 (got %d)", pr->chain_group);
  if (pr->prologue != GDN_PROLOGUE_NONE && pr->prologue != GDN_PROLOGUE_FEATURES)
    return fail(GDN_ERR_INVALID_ARGUMENT, "unknown prologue %d", pr->prologue);
  if (pr->intra != GDN_INTRA_SEQUENTIAL && pr->intra != GDN_INTRA_JACOBI)
    return fail(GDN_ERR_INVALID_ARGUMENT, "unknown intra %d", pr->intra);
  if (pr->batch < 1 || pr->heads < 1 || pr->frames < 1 || pr->tokens_per_frame < 1)
    return fail(GDN_ERR_INVALID_ARGUMENT, "batch, heads, frames and tokens_per_frame must be >= 1 "
                "(got %d, %d, %d, %d)", pr->batch, pr->heads, pr->frames, pr->tokens_per_frame);
  if (pr->d_k < 16 || pr->d_k > 128 || pr->d_k % 16 || pr->d_v < 16 || pr->d_v > 128 || pr->d_v % 16)
    return fail(GDN_ERR_INVALID_ARGUMENT, "d_k and d_v must be multiples of 16 in [16, 128] "
                "(got %d, %d)", pr->d_k, pr->d_v);
  if ((pr->qkv_dtype != GDN_F32 && pr->qkv_dtype != GDN_BF16) ||
      (pr->out_dtype != GDN_F32 && pr->out_dtype != GDN_BF16))
    return fail(GDN_ERR_INVALID_ARGUMENT, "qkv_dtype/out_dtype must be GDN_F32 or GDN_BF16");
  if (pr->algo != GDN_ALGO_AUTO && pr->algo != GDN_ALGO_CHUNKED && pr->algo != GDN_ALGO_RECURRENT)
    return fail(GDN_ERR_INVALID_ARGUMENT, "unknown algo %d", pr->algo);
  if (!std::isfinite(pr->key_scale))
    return fail(GDN_ERR_INVALID_ARGUMENT, "key_scale is not finite");
  if (direction >= 0 && direction != GDN_FORWARD && direction != GDN_BACKWARD &&
      direction != GDN_BIDIRECTIONAL && direction != GDN_CHUNK_CAUSAL)
    return fail(GDN_ERR_INVALID_ARGUMENT, "unknown direction %d", direction);
  if (direction == GDN_CHUNK_CAUSAL && (pr->first_chunk_frames < 1 || pr->chunk_frames < 1))
    return fail(GDN_ERR_INVALID_ARGUMENT, "GDN_CHUNK_CAUSAL needs first_chunk_frames and chunk_frames >= 1 "
                "(got %d, %d)", pr->first_chunk_frames, pr->chunk_frames);
  if (direction == GDN_CHUNK_CAUSAL && pr->intra == GDN_INTRA_JACOBI)
    return fail(GDN_ERR_UNSUPPORTED, "GDN_CHUNK_CAUSAL is built for the token-wise transition only");
  const long long T = (long long)pr->frames * pr->tokens_per_frame;
  // Element offsets are 64-bit in every kernel; keep each tensor well inside
  // the range the launch grids and workspace arithmetic assume.
  const long long rows = (long long)pr->batch * T * pr->heads;
  if (T > (1LL << 31) - 1 || rows * 128 > (1LL << 40))
    return fail(GDN_ERR_INVALID_ARGUMENT, "sequence too large (%lld tokens)", T);
  out->B = pr->batch;
  out->H = pr->heads;
  out->dk = pr->d_k;
  out->dv = pr->d_v;
  out->F = pr->frames;
  out->S = pr->tokens_per_frame;
  out->T = T;
  out->qkv_bf16 = pr->qkv_dtype == GDN_BF16;
  out->out_bf16 = pr->out_dtype == GDN_BF16;
  out->key_scale = pr->key_scale;
  out->jacobi = pr->intra == GDN_INTRA_JACOBI;
  out->first_chunk_frames = pr->first_chunk_frames;
  out->chunk_frames = pr->chunk_frames;
  out->prologue = pr->prologue == GDN_PROLOGUE_FEATURES;
  out->segment_tokens = pr->segment_tokens;
  out->chain_group = pr->chain_group;
  out->serial_scans = (pr->flags & GDN_FLAG_SERIAL_SCANS) != 0;
  out->tm_reuse = (pr->flags & GDN_FLAG_FORM_INVERSE) == 0;
  out->strip_scan = (pr->flags & GDN_FLAG_NO_STRIP_SCAN) == 0;
  return GDN_OK;
}

enum class Path { Recurrent, Chunked, Jacobi };

gdn_status choose_path(const gdn_problem* pr, const gdn::Problem& p, Path* path) {
  if (p.jacobi) {
    if (pr->algo == GDN_ALGO_RECURRENT)
      return fail(GDN_ERR_UNSUPPORTED, "the frame-level transition has no token-recurrent path");
    const char* why = gdn::jacobi_unsupported_reason(p);
    if (why) return fail(GDN_ERR_UNSUPPORTED, "frame-level path: %s", why);
    *path = Path::Jacobi;
    return GDN_OK;
  }
  if (pr->algo == GDN_ALGO_RECURRENT) { *path = Path::Recurrent; return GDN_OK; }
  if (pr->algo == GDN_ALGO_AUTO && !p.qkv_bf16) { *path = Path::Recurrent; return GDN_OK; }
  const char* why = gdn::chunked_unsupported_reason(p);
  if (why) {
    if (pr->algo == GDN_ALGO_CHUNKED) return fail(GDN_ERR_UNSUPPORTED, "chunked path: %s", why);
    *path = Path::Recurrent;
    return GDN_OK;
  }
  *path = Path::Chunked;
  return GDN_OK;
}

size_t workspace_for(Path path, const gdn::Problem& p, int direction) {
  return path == Path::Chunked  ? gdn::chunked_workspace(p, direction)
         : path == Path::Jacobi ? gdn::jacobi_workspace(p, direction)
                                : gdn::recurrent_workspace(p, direction);
}

gdn_status run(const gdn_problem* pr, int direction, const gdn::Tensors& t, void* workspace,
               size_t workspace_bytes, void* stream) {
  gdn::Problem p;
  gdn_status s = check_problem(pr, direction, &p);
  if (s != GDN_OK) return s;
  if (!t.q || !t.k || !t.v || !t.g || !t.beta || !t.out)
    return fail(GDN_ERR_INVALID_ARGUMENT, "q, k, v, log_gate, beta and out must be non-NULL");
  const void* ptrs[] = {t.q, t.k, t.v, t.g, t.beta, t.h0, t.out, t.hT, workspace};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr))
      return fail(GDN_ERR_INVALID_ARGUMENT, "tensor and workspace pointers must be 16-byte aligned");
  Path path;
  s = choose_path(pr, p, &path);
  if (s != GDN_OK) return s;
  const size_t need = workspace_for(path, p, direction);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(GDN_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes needed, %zu given%s", need,
                workspace_bytes, workspace ? "" : " (NULL)");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = path == Path::Chunked  ? gdn::chunked_launch(p, direction, t, workspace, st)
                 : path == Path::Jacobi ? gdn::jacobi_launch(p, direction, t, workspace, st)
                                        : gdn::recurrent_launch(p, direction, t, workspace, st);
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
  g_last_error.clear();
  return GDN_OK;
}

}  // namespace

extern "C" {

int32_t gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_status_string(gdn_status s) {
  switch (s) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_INVALID_ARGUMENT: return "GDN_ERR_INVALID_ARGUMENT";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
    case GDN_ERR_WORKSPACE_TOO_SMALL: return "GDN_ERR_WORKSPACE_TOO_SMALL";
    case GDN_ERR_HIP: return "GDN_ERR_HIP";
    default: return "GDN_ERR_UNKNOWN_STATUS";
  }
}

const char* gdn_last_error_message(void) { return g_last_error.c_str(); }

gdn_status gdn_plan_segment_tokens(const gdn_problem* pr, int32_t direction, int32_t* tokens_out) {
  try {
    if (!tokens_out) return fail(GDN_ERR_INVALID_ARGUMENT, "tokens_out is NULL");
    gdn::Problem p;
    gdn_status s = check_problem(pr, direction, &p);
    if (s != GDN_OK) return s;
    Path path;
    s = choose_path(pr, p, &path);
    if (s != GDN_OK) return s;
    *tokens_out = path == Path::Chunked ? gdn::chunked_segment_tokens(p, direction) : 0;
    g_last_error.clear();
    return GDN_OK;
  } catch (...) {
    return fail(GDN_ERR_INVALID_ARGUMENT, "internal error while planning");
  }
}

gdn_status gdn_workspace_size(const gdn_problem* pr, int32_t direction, size_t* bytes_out) {
  try {
    if (!bytes_out) return fail(GDN_ERR_INVALID_ARGUMENT, "bytes_out is NULL");
    gdn::Problem p;
    gdn_status s = check_problem(pr, direction, &p);
    if (s != GDN_OK) return s;
    Path path;
    s = choose_path(pr, p, &path);
    if (s != GDN_OK) return s;
    *bytes_out = workspace_for(path, p, direction);
    g_last_error.clear();
    return GDN_OK;
  } catch (...) {
    return fail(GDN_ERR_INVALID_ARGUMENT, "internal error while sizing the workspace");
  }
}

gdn_status gdn_forward(const gdn_problem* pr, int32_t direction, const void* q, const void* k,
                       const void* v, const float* log_gate, const float* beta,
                       const float* initial_state, void* out, float* final_state,
                       void* workspace, size_t workspace_bytes, void* stream) {
  try {
    gdn::Tensors t{q, k, v, log_gate, beta, initial_state, out, final_state};
    return run(pr, direction, t, workspace, workspace_bytes, stream);
  } catch (...) {
    return fail(GDN_ERR_HIP, "internal error while enqueueing");
  }
}

gdn_status gdn_step(const gdn_problem* pr, const void* q, const void* k, const void* v,
                    const float* log_gate, const float* beta, const float* state_in,
                    float* state_out, void* out, void* workspace, size_t workspace_bytes,
                    void* stream) {
  try {
    if (pr && pr->frames != 1)
      return fail(GDN_ERR_INVALID_ARGUMENT, "gdn_step takes exactly one frame (frames = %d)",
                  pr->frames);
    if (!state_out) return fail(GDN_ERR_INVALID_ARGUMENT, "state_out must be non-NULL");
    gdn::Tensors t{q, k, v, log_gate, beta, state_in, out, state_out};
    return run(pr, GDN_FORWARD, t, workspace, workspace_bytes, stream);
  } catch (...) {
    return fail(GDN_ERR_HIP, "internal error while enqueueing");
  }
}

gdn_status gdn_step_noalloc(const gdn_problem* pr, const void* q, const void* k, const void* v,
                            const float* log_gate, const float* beta, const float* state_in,
                            float* state_out, void* out, void* stream) {
  try {
    if (pr && pr->frames != 1)
      return fail(GDN_ERR_INVALID_ARGUMENT, "gdn_step_noalloc takes exactly one frame (frames = %d)",
                  pr->frames);
    if (!state_out) return fail(GDN_ERR_INVALID_ARGUMENT, "state_out must be non-NULL");
    // size the step on the host first: an oversized one is rejected before any HIP call
    gdn::Problem p;
    gdn_status s = check_problem(pr, GDN_FORWARD, &p);
    if (s != GDN_OK) return s;
    Path path;
    s = choose_path(pr, p, &path);
    if (s != GDN_OK) return s;
    const size_t need = workspace_for(path, p, GDN_FORWARD);
    if (need > (size_t)GDN_NOALLOC_SCRATCH_BYTES)
      return fail(GDN_ERR_WORKSPACE_TOO_SMALL,
                  "gdn_step_noalloc: this step needs %zu bytes of scratch, the library's static scratch "
                  "holds %zu; call gdn_step with a workspace instead", need, (size_t)GDN_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if (need > 0) {
      const hipError_t e = gdn::noalloc_scratch(&ws);
      if (e != hipSuccess) return fail(GDN_ERR_HIP, "HIP error taking the scratch address: %s", hipGetErrorString(e));
    }
    gdn::Tensors t{q, k, v, log_gate, beta, state_in, out, state_out};
    return run(pr, GDN_FORWARD, t, ws, need, stream);
  } catch (...) {
    return fail(GDN_ERR_HIP, "internal error while enqueueing");
  }
}

}  // extern "C"
