// Internal interface between the C-ABI layer (gdn_api.cpp) and the kernel
// launchers.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gdn.h"

namespace gdn {

// A validated problem with plain integer sizes.
struct Problem {
  int B, H, dk, dv, F, S;
  long long T;         // F * S
  bool qkv_bf16;       // q/k/v element type (else fp32)
  bool out_bf16;       // out element type (else fp32)
  float key_scale;
  bool jacobi;         // frame-level transition (GDN_INTRA_JACOBI)
  int first_chunk_frames, chunk_frames;   // GDN_CHUNK_CAUSAL chunking (frames)
  bool prologue;       // GDN_PROLOGUE_FEATURES
  int segment_tokens;  // 0: automatic
  int chain_group;     // 0: automatic, 1: whole, m >= 2: groups of m
  bool serial_scans;   // GDN_FLAG_SERIAL_SCANS
  bool tm_reuse;       // !GDN_FLAG_FORM_INVERSE
  bool strip_scan;     // !GDN_FLAG_NO_STRIP_SCAN
};

// Device pointers of one call.
struct Tensors {
  const void* q;
  const void* k;
  const void* v;
  const float* g;      // log-gate
  const float* beta;
  const float* h0;     // may be null (zeros)
  void* out;
  float* hT;           // may be null
};

// Token-sequential reference path (gdn_recurrent.hip).
size_t recurrent_workspace(const Problem& p, int direction);
hipError_t recurrent_launch(const Problem& p, int direction, const Tensors& t,
                            void* workspace, hipStream_t stream);

// Frame-chunked MFMA path (gdn_chunked.hip).
// Returns null when supported, else a static reason string.
const char* chunked_unsupported_reason(const Problem& p);
size_t chunked_workspace(const Problem& p, int direction);
hipError_t chunked_launch(const Problem& p, int direction, const Tensors& t,
                          void* workspace, hipStream_t stream);

// Frame-level (Jacobi) transition (gdn_chunked.hip).
const char* jacobi_unsupported_reason(const Problem& p);
size_t jacobi_workspace(const Problem& p, int direction);
hipError_t jacobi_launch(const Problem& p, int direction, const Tensors& t,
                         void* workspace, hipStream_t stream);

// Feature prologue (gdn_prologue.hip): two fp32 factors per (token, head) in
// the workspace, pairs (fk, fq) = (1/sqrt(mean k^2 + eps), 1/sqrt(sum q^2 + eps)):
// fac[2 i], fac[2 i + 1] with i = (b H + h)(T + 2) + t + 1 (a zero pair before
// token 0 and after token T - 1 of every (batch, head)).
size_t prologue_bytes(const Problem& p);
hipError_t prologue_launch(const Problem& p, const Tensors& t, float* fac, hipStream_t stream);

int chunked_segment_tokens(const Problem& p, int direction);

// Device address of the allocation-free step's scratch array on the current
// device (gdn_noalloc.hip; GDN_NOALLOC_SCRATCH_BYTES bytes, 256-byte aligned),
// taken once per device.
hipError_t noalloc_scratch(void** ptr);

// Kernel timing hooks (gdn_profile.cpp): no-ops unless profiling is enabled.
void prof_begin(hipStream_t stream, int kernel);
void prof_end(hipStream_t stream, int kernel);

// Round-up helper for workspace carving.
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace gdn
