/*
 * libgdn -- frame-wise gated delta rule (Gated DeltaNet) layer forward on
 * AMD Instinct MI355X (gfx950).  C ABI: plain pointers and sizes only.
 *
 * What is computed.  Per (batch b, head h) the layer carries a state
 * H in R^{d_k x d_v} (fp32).  For every token t of a frame-ordered sequence
 * (token t = f * tokens_per_frame + s, raster order inside a frame):
 *
 *     H   <- exp(g_t) * H                                  decay gate
 *     e   <- v_t - H^T (c k_t)                             value residual
 *     H   <- H + beta_t * (c k_t) e^T                      delta-rule write
 *     o_t  = H^T q_t                                       read after write
 *
 * with c = key_scale.  This is the token-wise Gated DeltaNet update of
 * "SANA-WM: Efficient Minute-Scale World Modeling with Hybrid Linear
 * Diffusion Transformer" (summary page), section 3.2 "Frame-wise Gated
 * DeltaNet (GDN)", token-wise update equation, written for the stored
 * orientation H = S^T (the page's S is d_v x d_k).  The sequence is scanned
 * one latent frame at a time with the state handed from frame to frame (same
 * section, frame-wise recurrence; "SANA-WM: a minute of camera-controlled
 * world, and where its memory actually lives", section "The linear part": 880
 * tokens per 704x1280 frame, 121 frames per minute, 112x112 state per head).
 *
 * Directions (same summary page, section 3.2 "Bidirectional and Chunk-Causal
 * GDN Variants"): GDN_FORWARD scans past -> future; GDN_BACKWARD scans the
 * whole token axis reversed (frames and the raster order inside frames);
 * GDN_BIDIRECTIONAL returns the sum of the two scans' outputs, the forward
 * scan starting from initial_state and the reversed scan from zero.
 *
 * Layouts (all tensors dense, row-major, caller-owned DEVICE memory):
 *   q, k        [B, T, H, d_k]    qkv_dtype (fp32 or bf16)
 *   v           [B, T, H, d_v]    qkv_dtype
 *   log_gate    [B, T, H]         fp32, g_t <= 0 on the documented domain
 *   beta        [B, T, H]         fp32, in [0, 1] on the documented domain
 *   states      [B, H, d_k, d_v]  fp32, element [b][h][i][j] maps key
 *                                 component i to value component j
 *   out         [B, T, H, d_v]    out_dtype
 * with T = frames * tokens_per_frame.  Every tensor pointer must be 16-byte
 * aligned.
 *
 * Calls are asynchronous on `stream` (a hipStream_t; NULL = the null stream)
 * and return after enqueueing.  `stream` must belong to the current device.
 * A bidirectional or chunk-causal call of the chunked path also runs part of
 * its work on a stream the library owns (see GDN_FLAG_SERIAL_SCANS), joined
 * back into `stream` with events before the call's last kernel.  The library
 * keeps no other state between calls and allocates no device memory: the
 * caller passes a workspace of at least gdn_workspace_size() bytes.  All
 * arguments are validated on the host before anything is enqueued; on any
 * error nothing is enqueued and a status other than GDN_OK is returned, with
 * a description available from gdn_last_error_message() on the same thread.
 * Input values are not checked: outside the documented domain, and for
 * NaN/Inf inputs, values propagate.  No C++ exception crosses this boundary
 * and the library never prints.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 2

typedef int32_t gdn_status;
enum {
  GDN_OK = 0,
  GDN_ERR_INVALID_ARGUMENT = 1,     /* null pointer, bad size, bad enum, misalignment */
  GDN_ERR_UNSUPPORTED = 2,          /* valid request this library does not implement */
  GDN_ERR_WORKSPACE_TOO_SMALL = 3,  /* workspace_bytes < gdn_workspace_size() */
  GDN_ERR_HIP = 4                   /* a HIP runtime call or kernel launch failed */
};

enum { GDN_F32 = 0, GDN_BF16 = 1 };                                   /* tensor dtypes */
/* Directions.  CHUNK_CAUSAL: the forward scan over the whole sequence plus,
 * for every chunk of frames, a reversed scan confined to that chunk and
 * started from zero, outputs summed; the final state is the forward scan's
 * ("SANA-WM ... Hybrid Linear Diffusion Transformer" summary, section 3.2,
 * "Bidirectional and Chunk-Causal GDN Variants").  The chunks are
 * first_chunk_frames frames, then chunk_frames frames each (the last may be
 * shorter); see gdn_problem. */
enum { GDN_FORWARD = 0, GDN_BACKWARD = 1, GDN_BIDIRECTIONAL = 2, GDN_CHUNK_CAUSAL = 3 };

/* Algorithm selection.  AUTO picks the frame-chunked MFMA path for bf16 q/k/v
 * and the token-recurrent fp32 path for fp32 q/k/v (whose tolerance needs fp32
 * products).  RECURRENT forces the token-sequential kernel (any dtype).
 *
 * Numeric domain of the chunked path (AUTO with bf16 q/k/v, or CHUNKED).  Its
 * matrix-core products take fp16 operands with fp32 accumulation; states,
 * gates and accumulations are fp32.
 *   - Inputs: each bf16 value of q and k is converted to fp16 rounding
 *     toward zero.  That is exact for magnitudes in [2^-14, 65504] (a bf16
 *     value there has at most 8 significant bits, fp16 keeps 11), loses less
 *     than 2^-24 in absolute value below 2^-14, and saturates at +-65504
 *     above: such an input is taken as +-65504.  (With the feature prologue
 *     the normalised q and k, at most sqrt(d_k) in magnitude, are rounded to
 *     the nearest fp16.)  key_scale, the gates and beta enter as fp32
 *     factors.  v enters an fp32 residual exactly (the frame-level
 *     transition rounds c beta v to the nearest fp16).
 *   - Intermediates: the state, the per-token residuals v - prediction and
 *     the corrections they become after the sub-chunk's triangular solve,
 *     and (bidirectional and chunk-causal calls) the first scan's outputs,
 *     which are kept as an fp16 partial sum, are rounded to the nearest fp16
 *     at each product; a magnitude above 65504 there becomes +-inf and
 *     propagates.
 *   - Hence the chunked path is accurate (within 2e-2 of the output RMS)
 *     when every element of v, of the initial state and of each scan's
 *     outputs stays below 2^15 in magnitude.  On the documented domain
 *     (g <= 0, beta in [0, 1], |key_scale k| <= 1) the state and the
 *     corrections stay within a small multiple of max|v| + max|initial
 *     state|, so |v| and |initial state| up to about 2^12 keep every
 *     intermediate in range.  Larger magnitudes need GDN_ALGO_RECURRENT,
 *     which computes in fp32 throughout and has no such limit. */
enum { GDN_ALGO_AUTO = 0, GDN_ALGO_CHUNKED = 1, GDN_ALGO_RECURRENT = 2 };

/* Transition inside a frame.  SEQUENTIAL: the token-wise rule applied to every
 * token in order ("SANA-WM ... Hybrid Linear Diffusion Transformer" summary,
 * section 3.2, token-wise update).  JACOBI: the same page's frame-wise update,
 * in which every token of a frame reads the frame's end state:
 *   H_end = gamma (I - c^2 K^T diag(beta) K) H + c K^T diag(beta) V,  O = Q H_end
 * (stored orientation, c = key_scale) with one decay per frame, gamma =
 * exp(log_gate) of the frame's first token in the scan's order (the last
 * token of the frame for the reversed scan).  JACOBI runs on the chunked
 * machinery only: bf16 q/k/v, d_k = d_v <= 112, algo AUTO or CHUNKED. */
enum { GDN_INTRA_SEQUENTIAL = 0, GDN_INTRA_JACOBI = 1 };

/* Feature prologue applied to q and k on load.  NONE: q and k are used as
 * given.  FEATURES: per token and head, the key is replaced by its features
 * ReLU(RMSNorm(k)), k_i / sqrt(mean_j k_j^2 + 1e-6) with negative values set
 * to zero and no learned weight, and the query by q / sqrt(sum_j q_j^2 +
 * 1e-6); key_scale still multiplies the key features (the pages' spatial
 * scale is key_scale = 1/sqrt(d_k * tokens_per_frame)).  "SANA-WM ... Hybrid
 * Linear Diffusion Transformer" summary, section 3.2, "Algebraic
 * Stabilization for Spatial Token Explosion" (RMS-normalised, ReLU-activated
 * keys) and the token-wise update (normalised queries).  The normalised
 * tensors are never written to memory: a first kernel reads q and k once and
 * stores two fp32 factors per (token, head) in the workspace, and every
 * kernel that loads q or k applies them (and the ReLU) as it loads.  Every
 * path and direction supports it; the workspace grows by 8 * B * H * (T + 2)
 * bytes. */
enum { GDN_PROLOGUE_NONE = 0, GDN_PROLOGUE_FEATURES = 1 };

typedef struct gdn_problem {
  int32_t abi_version;        /* must equal GDN_ABI_VERSION */
  int32_t batch;              /* B >= 1 */
  int32_t heads;              /* H >= 1 */
  int32_t d_k;                /* key/query width: multiple of 16, <= 128 */
  int32_t d_v;                /* value width: multiple of 16, <= 128 */
  int32_t frames;             /* F >= 1 */
  int32_t tokens_per_frame;   /* S >= 1; T = F * S */
  int32_t qkv_dtype;          /* GDN_F32 or GDN_BF16 */
  int32_t out_dtype;          /* GDN_F32 or GDN_BF16 */
  int32_t algo;               /* GDN_ALGO_* */
  float key_scale;            /* keys are multiplied by this on load (finite) */
  int32_t intra;              /* GDN_INTRA_* (0 = SEQUENTIAL) */
  int32_t first_chunk_frames; /* GDN_CHUNK_CAUSAL: frames of the first chunk (>= 1), else ignored */
  int32_t chunk_frames;       /* GDN_CHUNK_CAUSAL: frames of each later chunk (>= 1), else ignored */
  int32_t prologue;           /* GDN_PROLOGUE_* (0 = NONE) */
  /* Tuning of the chunked and frame-level paths (0 = the default).  They are
   * part of the call's problem, so the plan and gdn_workspace_size() depend
   * only on the arguments of the call; results do not depend on them beyond
   * rounding (GDN_FLAG_* below: not at all). */
  int32_t segment_tokens;     /* chunked path: tokens per segment, rounded up to
                                 a multiple of 64; 0 = automatic (about five
                                 rounds of workgroups over the compute units,
                                 at most about 2 sqrt(T / 64) segments) */
  int32_t chain_group;        /* chain of segment (or frame) maps: 0 = automatic
                                 (a chain of 16 or more maps is split into groups
                                 of about sqrt(maps / 2): the groups' maps are
                                 composed in parallel, the group maps chained,
                                 each group expanded from its start state); 1 =
                                 never split; m >= 2 = groups of m maps whenever
                                 the chain is longer than m.  Bidirectional calls
                                 of the chunked path never split. */
  int32_t flags;              /* GDN_FLAG_* bits, see below; 0 = default */
  int32_t reserved[5];        /* must be zero */
} gdn_problem;

/* gdn_problem.flags.
 * SERIAL_SCANS: a bidirectional or chunk-causal call of the chunked path runs
 *   every kernel on the caller's stream, in order.  By default it forks part
 *   of its work onto a second stream that the library owns (one per caller
 *   stream, up to eight per device, created on first use with the default
 *   priority and kept until the process ends; a call whose stream finds no
 *   free one runs in order) and joins it back with events before its last
 *   kernel.  Results are bit-identical either way.
 * FORM_INVERSE: the output kernel of a forward- or backward-only call forms
 *   each 64-token sub-chunk's triangular inverse Tm diag(beta) itself instead
 *   of loading the one the scan's segment-map kernel formed (5 KB of fp16 per
 *   sub-chunk and head in the workspace, allocated either way).  Results are
 *   bit-identical (the same arithmetic on the same rows).  Two-scan calls and
 *   calls with a single segment always form it.
 * NO_STRIP_SCAN: a forward- or backward-only call of the chunked path with at
 *   most 32 sub-chunks of 64 tokens per head (T <= 2048; one streaming frame)
 *   runs through segment maps and their chain like longer calls.  By default
 *   such a call (without the feature prologue) takes the strip scan instead:
 *   one launch prepares every sub-chunk (its triangular inverse, its
 *   intra-chunk product and gate factors: 11008 bytes per sub-chunk and head
 *   in the workspace) and one runs the sub-chunks in order with a workgroup
 *   per 16 value columns of the state and head (the state's columns evolve
 *   independently).  Same algebra and rounding points; results agree to
 *   rounding (sums in another order). */
enum { GDN_FLAG_SERIAL_SCANS = 1, GDN_FLAG_FORM_INVERSE = 2, GDN_FLAG_NO_STRIP_SCAN = 4 };

/* Version of this ABI (GDN_ABI_VERSION of the built library). */
int32_t gdn_abi_version(void);

/* Static, never-NULL text for a status code. */
const char* gdn_status_string(gdn_status status);

/* Detail of the last non-OK status returned on the calling thread ("" if none).
 * The pointer stays valid until the next libgdn call on that thread. */
const char* gdn_last_error_message(void);

/* Bytes of device workspace gdn_forward needs for (problem, direction).
 * Pure host computation.  Errors as gdn_forward's argument checks. */
gdn_status gdn_workspace_size(const gdn_problem* problem, int32_t direction,
                              size_t* bytes_out);

/* Whole-sequence layer forward (offline / bidirectional mode).
 *   direction      GDN_FORWARD, GDN_BACKWARD or GDN_BIDIRECTIONAL
 *   initial_state  [B,H,d_k,d_v] fp32 or NULL (= zeros); seeds the forward scan
 *                  (the reversed scan in GDN_BACKWARD mode)
 *   final_state    [B,H,d_k,d_v] fp32 or NULL; receives the state after the
 *                  last token of the forward scan (of the reversed scan in
 *                  GDN_BACKWARD mode).  May alias initial_state; no other
 *                  aliasing between arguments is allowed.
 *   workspace      device scratch of workspace_bytes >= gdn_workspace_size();
 *                  may be NULL when that size is 0.  Its contents on entry are
 *                  ignored; it must not be used by anything else until the
 *                  enqueued work has finished.
 * Pages: the direction combination is the summary page's section 3.2,
 * "Bidirectional and Chunk-Causal GDN Variants" (independent scans, outputs
 * summed). */
gdn_status gdn_forward(const gdn_problem* problem, int32_t direction,
                       const void* q, const void* k, const void* v,
                       const float* log_gate, const float* beta,
                       const float* initial_state,
                       void* out, float* final_state,
                       void* workspace, size_t workspace_bytes,
                       void* stream);

/* One frame of the chunk-causal streaming forward scan with the state carried
 * between calls (summary page, section 3.2: in chunk-causal inference the
 * forward scan stays global; the state is the only thing passed on).
 *   problem->frames must be 1 (GDN_ERR_INVALID_ARGUMENT otherwise).
 *   state_in   [B,H,d_k,d_v] fp32 or NULL (= zeros)
 *   state_out  [B,H,d_k,d_v] fp32, required; may alias state_in (in place).
 *   workspace  as gdn_forward with GDN_FORWARD.
 * Calling it once per frame with state_out fed back as state_in reproduces
 * gdn_forward(GDN_FORWARD) over the concatenated frames. */
gdn_status gdn_step(const gdn_problem* problem,
                    const void* q, const void* k, const void* v,
                    const float* log_gate, const float* beta,
                    const float* state_in, float* state_out,
                    void* out,
                    void* workspace, size_t workspace_bytes,
                    void* stream);

/* Allocation-free variant of gdn_step, for callers that cannot allocate
 * device memory or hand over a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Arguments, results and
 * kernels are gdn_step's; in place of a workspace it uses a scratch array of
 * GDN_NOALLOC_SCRATCH_BYTES that is part of the library's code object (each
 * device the library runs on holds its own copy until the process ends; the
 * first call on a device takes the copy's address).  It allocates nothing.
 *   GDN_ERR_WORKSPACE_TOO_SMALL, with nothing enqueued, when the step's
 *   gdn_workspace_size(problem, GDN_FORWARD) exceeds the scratch (one
 *   880-token frame of 20 heads x 112 needs about 3 MB; at that width steps
 *   of up to 5120 tokens fit).
 * Every call on a device shares that device's scratch, which keeps the last
 * call's contents (nothing in it has to start at zero): calls that overlap on
 * one device (different streams, or threads without ordering) race on it and
 * must be serialised by the caller; calls on one stream are ordered. */
#define GDN_NOALLOC_SCRATCH_BYTES (64u << 20)
gdn_status gdn_step_noalloc(const gdn_problem* problem,
                            const void* q, const void* k, const void* v,
                            const float* log_gate, const float* beta,
                            const float* state_in, float* state_out,
                            void* out, void* stream);

/* Kernel timing (diagnostics).  While enabled, every kernel launch made by
 * libgdn is bracketed by two HIP events recorded on the call's stream;
 * gdn_profile_read() waits for the recorded events and returns, per kernel,
 * the number of launches and their summed duration in milliseconds since the
 * last reset.  Process-wide; intended for one measuring thread. */
enum {
  GDN_KERNEL_SEG_MAP = 0,     /* chunked path: per-segment affine state maps */
  GDN_KERNEL_SEG_CHAIN = 1,   /* chunked path: serial chain of segment maps */
  GDN_KERNEL_SEG_OUT = 2,     /* chunked path: outputs and final state */
  GDN_KERNEL_RECURRENT = 3,   /* token-sequential path */
  GDN_KERNEL_JAC_MAP = 4,     /* frame-level path: per-frame maps */
  GDN_KERNEL_JAC_OUT = 5,     /* frame-level path: outputs and final state */
  GDN_KERNEL_PROLOGUE = 6,    /* feature prologue: per-token key and query factors */
  GDN_KERNEL_SCAN_PREP = 7,   /* strip scan: per-sub-chunk inverses, intra-chunk products, gate factors */
  GDN_KERNEL_SCAN = 8,        /* strip scan: sub-chunks in order per state strip; outputs and final state */
  GDN_KERNEL_COUNT = 9
};
gdn_status gdn_profile_enable(int32_t on);
gdn_status gdn_profile_reset(void);
gdn_status gdn_profile_read(int32_t kernel, int64_t* launches, double* total_ms);
const char* gdn_kernel_name(int32_t kernel);   /* static text; "" if unknown */

/* Tokens per segment the chunked path would use for (problem, direction), or
 * 0 when the call would take the token-recurrent path.  Host only. */
gdn_status gdn_plan_segment_tokens(const gdn_problem* problem, int32_t direction, int32_t* tokens_out);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* GDN_H_ */
