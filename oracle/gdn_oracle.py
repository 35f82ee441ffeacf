"""CPU oracle for the frame-wise gated delta rule layer forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The GPU library
never calls it and shares no code with it.

Plain, slow, float64, single-threaded NumPy.  Every input is widened exactly to
float64 (bf16 and fp32 values are exactly representable), so the oracle sees
precisely the values the GPU receives.

Pages cited (by title):
  [WM-summary]  "SANA-WM: Efficient Minute-Scale World Modeling with Hybrid
                Linear Diffusion Transformer" (structured paper summary),
                section "Memory-Efficient Long-Context Modeling (Section 3.2)".
  [WM-teardown] "SANA-WM: a minute of camera-controlled world, and where its
                memory actually lives", section "The linear part: a gated delta
                rule, one frame per step".

Notation and layout.  For one (batch, head): q_t, k_t in R^{d_k}, v_t in
R^{d_v}, log-gate g_t (the decay gate is gamma_t = exp(g_t) in (0, 1]), write
strength beta_t.  The pages write the state as S in R^{d_v x d_k}; this module
stores its transpose H = S^T in R^{d_k x d_v}, so that o = H^T q, i.e.
o_j = sum_i q_i H[i, j].  Tensors: q, k [B,T,H,d_k]; v [B,T,H,d_v];
log_gate, beta [B,T,H]; states [B,H,d_k,d_v].  Token t = f*S + s (frame-major).

Readings taken where the pages are silent or ambiguous:
  * Within a frame the update is the token-wise rule applied to each token in
    raster order (frame-major token axis), and the state is handed from frame
    to frame ("Reading A").  The pages' literal frame-level transition is kept
    as ``jacobi`` ("Reading B").
  * The output reads the state after the token's own write (o_i = S_i q_i).
  * The reversed-time scan reverses the whole token axis (frame order and the
    order inside each frame), starting from a zero state; the bidirectional
    output is the plain sum of the two scans; the final state reported is the
    forward scan's.
  * ``key_scale`` multiplies every key before use (1.0 = keys as given); the
    pages' spatial key scale is 1/sqrt(D*S) on RMS-normalised keys, which for
    unit-norm keys is 1/sqrt(S).
  * Feature prologue (``key_features``, ``query_features``): the key features
    are ReLU of the key RMS-normalised over its d_k components, per token and
    head, with no learned weight (the pages give none) and
    ``PROLOGUE_EPS`` added to the mean square; the queries are
    L2-normalised per token and head with ``PROLOGUE_EPS`` added to the sum of
    squares (the pages call them normalised queries without saying how; unit
    L2 norm is the token-wise Gated DeltaNet practice they refer to).  The
    spatial scale 1/sqrt(D*S) stays the separate ``key_scale``.
"""
from __future__ import annotations

import numpy as np

__all__ = ["fwd", "bwd", "bidir", "step", "jacobi", "jacobi_bwd", "jacobi_bidir", "forward",
           "jacobi_forward", "chunk_causal", "chunk_bounds", "key_features", "query_features",
           "PROLOGUE_EPS"]

PROLOGUE_EPS = 1e-6


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def key_features(k, eps=PROLOGUE_EPS):
    """Key features before the spatial scale: ReLU(RMSNorm(k)).

    [WM-summary] section 3.2, "Algebraic Stabilization for Spatial Token
    Explosion": the keys are RMS-normalised and ReLU-activated, so a key's
    squared norm is about d_k, before the 1/sqrt(D*S) scale.  Per token and
    head over the last axis:
        kbar = max(k / sqrt(mean(k^2) + eps), 0)
    NaN inputs stay NaN.
    """
    k = _as64(k)
    rms = np.sqrt(np.mean(k * k, axis=-1, keepdims=True) + eps)
    return np.maximum(k / rms, 0.0)


def query_features(q, eps=PROLOGUE_EPS):
    """Normalised queries: q / sqrt(sum(q^2) + eps) per token and head.

    [WM-summary] section 3.2, "Frame-wise Gated DeltaNet (GDN)": the update
    reads the state with the normalised query; the token-wise Gated DeltaNet
    normalises queries (and keys) to unit L2 norm ("Algebraic Stabilization
    for Spatial Token Explosion", on the standard 1/sqrt(D) normalisation).
    """
    q = _as64(q)
    return q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + eps)


def fwd(q, k, v, log_gate, beta, h0=None, key_scale=1.0):
    """Forward scan of the token-wise gated delta rule.

    [WM-summary] section 3.2, "Frame-wise Gated DeltaNet (GDN)", token-wise
    update: decay the state by gamma_i, predict the value with the key,
    write the beta-gated residual as a rank-1 update, then read with the
    query.  In the stored orientation H = S^T, per token:
        H <- gamma_t * H
        e <- v_t - H^T k_t            (the "surprise")
        H <- H + beta_t * k_t e^T
        o_t = H^T q_t
    Returns (o [B,T,H,d_v] float64, final state [B,H,d_k,d_v] float64).
    """
    q, k, v = _as64(q), _as64(k) * float(key_scale), _as64(v)
    g, b = _as64(log_gate), _as64(beta)
    B, T, Hh, dk = q.shape
    dv = v.shape[-1]
    H = np.zeros((B, Hh, dk, dv)) if h0 is None else _as64(h0).copy()
    o = np.zeros((B, T, Hh, dv))
    for t in range(T):
        kt = k[:, t]                                   # [B,H,dk]
        H *= np.exp(g[:, t])[:, :, None, None]         # gamma_t * S_{t-1}
        pred = np.einsum("bhi,bhij->bhj", kt, H)       # S_{t-1} gamma k (stored: H^T k)
        e = v[:, t] - pred
        H += b[:, t][:, :, None, None] * kt[:, :, :, None] * e[:, :, None, :]
        o[:, t] = np.einsum("bhi,bhij->bhj", q[:, t], H)
    return o, H


def bwd(q, k, v, log_gate, beta, h0=None, key_scale=1.0):
    """Reversed-time scan: the forward scan over the token axis reversed.

    [WM-summary] section 3.2, "Bidirectional and Chunk-Causal GDN Variants":
    a reversed-time scan runs future -> past.  Reading: the whole token axis
    is reversed (frames and the raster order inside each frame).  ``h0``
    seeds the reversed scan; the state returned is the state after token 0.
    """
    flip = lambda x: np.flip(_as64(x), axis=1)
    o, H = fwd(flip(q), flip(k), flip(v), flip(log_gate), flip(beta), h0, key_scale)
    return np.flip(o, axis=1).copy(), H


def bidir(q, k, v, log_gate, beta, h0=None, key_scale=1.0):
    """Bidirectional layer: forward scan plus reversed scan, outputs summed.

    [WM-summary] section 3.2, "Bidirectional and Chunk-Causal GDN Variants":
    the two scans are computed independently and their outputs summed.  The
    forward scan starts from ``h0``, the reversed scan from zero; the final
    state is the forward scan's.
    """
    of, Hf = fwd(q, k, v, log_gate, beta, h0, key_scale)
    ob, _ = bwd(q, k, v, log_gate, beta, None, key_scale)
    return of + ob, Hf


def chunk_bounds(frames, first_chunk_frames, chunk_frames):
    """Frame ranges [f0, f1) of the chunks: the first holds
    ``first_chunk_frames`` frames, every later one ``chunk_frames`` (the last
    may hold fewer)."""
    out, f0 = [], 0
    n = first_chunk_frames
    while f0 < frames:
        f1 = min(frames, f0 + n)
        out.append((f0, f1))
        f0, n = f1, chunk_frames
    return out


def chunk_causal(q, k, v, log_gate, beta, h0=None, key_scale=1.0, tokens_per_frame=None,
                 first_chunk_frames=1, chunk_frames=1):
    """Chunk-causal layer: a global forward scan from ``h0`` plus, for every
    chunk of frames, a reversed scan over that chunk alone from a zero state;
    outputs summed, final state the forward scan's.

    [WM-summary] section 3.2, "Bidirectional and Chunk-Causal GDN Variants":
    in chunk-causal mode the forward scan stays global while the reversed
    scan is confined to the current chunk.  Chunk sizes (in latent frames)
    follow the streaming release: a first chunk, then equal chunks.
    """
    T = np.asarray(q).shape[1]
    S = T if tokens_per_frame is None else int(tokens_per_frame)
    if T % S:
        raise ValueError("token count is not a whole number of frames")
    o, H = fwd(q, k, v, log_gate, beta, h0, key_scale)
    for f0, f1 in chunk_bounds(T // S, first_chunk_frames, chunk_frames):
        sl = slice(f0 * S, f1 * S)
        ob, _ = bwd(*(np.asarray(x)[:, sl] for x in (q, k, v, log_gate, beta)), None, key_scale)
        o[:, sl] += ob
    return o, H


def step(q, k, v, log_gate, beta, state_in, key_scale=1.0):
    """One frame of the chunk-causal forward scan with the state carried.

    [WM-summary] section 3.2, "Bidirectional and Chunk-Causal GDN Variants":
    in chunk-causal inference the forward scan stays global, so each new
    frame continues from the carried state.  Returns (o, state_out).
    """
    return fwd(q, k, v, log_gate, beta, state_in, key_scale)


def jacobi(q, k, v, log_gate, beta, h0=None, key_scale=1.0, tokens_per_frame=None):
    """The pages' literal frame-level transition (Reading B).

    [WM-summary] section 3.2, "Frame-wise Gated DeltaNet (GDN)", frame-wise
    update: S_t = S_{t-1} M_t + U_t with M_t = gamma_t (I - K_t beta_t K_t^T),
    U_t = V_t beta_t K_t^T and O_t = S_t Q_t.  In the stored orientation:
        H <- gamma H + K^T diag(beta) (V - gamma K H);   O = Q H
    The frame decay gamma_t is taken from the gate of the frame's first token
    (the pages give one scalar per frame).  Every token of the frame reads the
    end-of-frame state.
    """
    q, k, v = _as64(q), _as64(k) * float(key_scale), _as64(v)
    g, b = _as64(log_gate), _as64(beta)
    B, T, Hh, dk = q.shape
    dv = v.shape[-1]
    S = T if tokens_per_frame is None else int(tokens_per_frame)
    if T % S:
        raise ValueError("token count is not a whole number of frames")
    H = np.zeros((B, Hh, dk, dv)) if h0 is None else _as64(h0).copy()
    o = np.zeros((B, T, Hh, dv))
    for f in range(T // S):
        sl = slice(f * S, (f + 1) * S)
        Kf = k[:, sl].transpose(0, 2, 1, 3)             # [B,H,S,dk]
        Vf = v[:, sl].transpose(0, 2, 1, 3)             # [B,H,S,dv]
        Qf = q[:, sl].transpose(0, 2, 1, 3)
        bf = b[:, sl].transpose(0, 2, 1)                # [B,H,S]
        gamma = np.exp(g[:, f * S])[:, :, None, None]   # [B,H,1,1]
        resid = Vf - gamma * (Kf @ H)                   # V - gamma K H
        H = gamma * H + np.swapaxes(Kf, -1, -2) @ (bf[..., None] * resid)
        o[:, sl] = (Qf @ H).transpose(0, 2, 1, 3)
    return o, H


def jacobi_bwd(q, k, v, log_gate, beta, h0=None, key_scale=1.0, tokens_per_frame=None):
    """Reversed-time scan of the frame-level transition.

    [WM-summary] section 3.2, "Bidirectional and Chunk-Causal GDN Variants",
    applied to the frame-wise update: the reversed scan is the forward scan of
    the reversed token axis, so frames are visited last to first and a frame's
    decay is the gate of its last token (the first one the reversed scan
    meets).  ``h0`` seeds the reversed scan; the state returned is the state
    after frame 0.
    """
    flip = lambda x: np.flip(_as64(x), axis=1)
    o, H = jacobi(flip(q), flip(k), flip(v), flip(log_gate), flip(beta), h0, key_scale, tokens_per_frame)
    return np.flip(o, axis=1).copy(), H


def jacobi_bidir(q, k, v, log_gate, beta, h0=None, key_scale=1.0, tokens_per_frame=None):
    """Bidirectional layer with the frame-level transition: the forward scan
    from ``h0`` plus the reversed scan from zero, outputs summed; the final
    state is the forward scan's ([WM-summary] section 3.2, "Bidirectional and
    Chunk-Causal GDN Variants")."""
    of, Hf = jacobi(q, k, v, log_gate, beta, h0, key_scale, tokens_per_frame)
    ob, _ = jacobi_bwd(q, k, v, log_gate, beta, None, key_scale, tokens_per_frame)
    return of + ob, Hf


def jacobi_forward(direction, q, k, v, log_gate, beta, h0=None, key_scale=1.0, tokens_per_frame=None):
    """Dispatch of the frame-level transition by direction name."""
    fn = {"fwd": jacobi, "bwd": jacobi_bwd, "bidir": jacobi_bidir}[direction]
    return fn(q, k, v, log_gate, beta, h0, key_scale, tokens_per_frame)


def forward(direction, q, k, v, log_gate, beta, h0=None, key_scale=1.0):
    """Dispatch by direction name: "fwd", "bwd" or "bidir"."""
    fn = {"fwd": fwd, "bwd": bwd, "bidir": bidir}[direction]
    return fn(q, k, v, log_gate, beta, h0, key_scale)
