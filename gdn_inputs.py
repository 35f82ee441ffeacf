"""Seeded synthetic inputs for the frame-wise gated delta rule layer.

This module draws random tensors with the shapes, value distributions and
structure of the layer's workloads.  It holds none of the recurrence's
arithmetic: both the CPU oracle (``oracle/``) and the GPU path consume what it
returns, and neither imports the other.

Workload shapes come from the SANA-WM pages:
  * "SANA-WM: a minute of camera-controlled world, and where its memory
    actually lives", section "Why a minute is hard: count the tokens": a
    704x1280 latent frame is a 22x40 grid of 880 tokens, a 60 s clip is 121
    latent frames (106,480 tokens);
  * same page, section "The linear part": 20 heads with a 112x112 fp32 state.
The trained weights, clips and benchmark scenes are not available, so every
tensor here is synthetic (see ``WORKLOADS`` for each recipe).

Recipe (all draws from one ``numpy.random.Generator(PCG64(seed))``, in this
order): q, k ~ N(0,1) then L2-normalised per (b, t, h); v ~ N(0,1);
u ~ U(lo, hi) with log-gate g = -u (per token, or per (b, frame, h) and shared
by the frame's tokens); beta = sigmoid(sigma_beta * N(0,1)); initial state
h0 = sigma_h0 * N(0,1) only when sigma_h0 > 0 (otherwise zeros, no draw).
Raw projections (``qk_spread`` > 0, the inputs of the feature prologue): q and
k are not normalised; after h0, m_q and m_k ~ N(0,1) per (b, t, h) are drawn
and q, k are multiplied by exp(qk_spread * m_q), exp(qk_spread * m_k), so
that token magnitudes vary over about a decade.
For bf16 workloads q, k, v are then rounded to bf16 (round to nearest even)
once; every consumer receives exactly those values.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    """Shape and distribution recipe of one synthetic workload."""

    name: str
    batch: int
    heads: int
    d_k: int
    d_v: int
    frames: int
    tokens_per_frame: int
    qkv_dtype: str            # "f32" or "bf16"; gates, beta and states are fp32
    gate_lo: float            # log-gate g = -U(gate_lo, gate_hi)
    gate_hi: float
    gate_per_frame: bool      # one gate per (b, frame, h), shared by the frame
    beta_sigma: float         # beta = sigmoid(beta_sigma * N(0,1))
    h0_sigma: float           # initial state ~ h0_sigma * N(0,1); 0 -> zeros
    mode: str                 # how the layer is run on it: "bidir" or "step"
    description: str = ""
    qk_spread: float = 0.0    # > 0: raw (unnormalised) q, k with log-normal token magnitudes

    @property
    def tokens(self) -> int:
        return self.frames * self.tokens_per_frame

    def resized(self, **kw) -> "Workload":
        """Same distributions, other sizes (for small parity cases)."""
        return dataclasses.replace(self, **kw)


# Index i matches the i-th workload of the layer's benchmark list.
WORKLOADS = [
    Workload("tiny_3x16_d16", 1, 1, 16, 16, 3, 16, "f32", 0.01, 0.2, False, 1.0, 0.0,
             "bidir", "tiny oracle check: 3 frames of a 4x4 grid, d=16, fp32"),
    Workload("clip5s_21x880_h20d112", 1, 20, 112, 112, 21, 880, "bf16", 0.001, 0.1, False,
             1.0, 0.0, "bidir", "5 s clip, bidirectional layer forward"),
    Workload("clip60s_121x880_h20d112", 1, 20, 112, 112, 121, 880, "bf16", 0.001, 0.1, False,
             1.0, 0.0, "bidir", "60 s 720p layer forward"),
    Workload("stream60s_121x880_h20d112", 1, 20, 112, 112, 121, 880, "bf16", 0.0005, 0.02,
             False, 1.0, 0.0, "step", "chunk-causal streaming: 121 one-frame steps"),
    Workload("batched_b2_121x880_h35d64", 2, 35, 64, 64, 121, 880, "bf16", 0.001, 0.1, True,
             2.0, 0.1, "bidir", "batch 2, 35 heads x 64, frame-shared gates"),
]


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32.

    Finite inputs only (the generator never produces NaN or Inf).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = ((bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return rounded.astype(np.uint32).view(np.float32)


def _l2_normalise(x: np.ndarray) -> np.ndarray:
    x64 = x.astype(np.float64)
    n = np.sqrt(np.sum(x64 * x64, axis=-1, keepdims=True))
    return (x64 / n).astype(np.float32)


def make_inputs(w: Workload, seed: int = 0) -> dict:
    """Draw one seeded input set for workload ``w``.

    Returns float32 numpy arrays in the library's layouts:
      q, k: [B, T, H, d_k]; v: [B, T, H, d_v]; log_gate, beta: [B, T, H];
      h0: [B, H, d_k, d_v].
    For bf16 workloads q, k, v hold bf16-representable values (float32 storage).
    """
    B, H, T, F, S = w.batch, w.heads, w.tokens, w.frames, w.tokens_per_frame
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((B, T, H, w.d_k), dtype=np.float32)
    k = rng.standard_normal((B, T, H, w.d_k), dtype=np.float32)
    if w.qk_spread <= 0:
        q, k = _l2_normalise(q), _l2_normalise(k)
    v = rng.standard_normal((B, T, H, w.d_v), dtype=np.float32)
    if w.gate_per_frame:
        u = rng.uniform(w.gate_lo, w.gate_hi, (B, F, H))
        u = np.repeat(u, S, axis=1)
    else:
        u = rng.uniform(w.gate_lo, w.gate_hi, (B, T, H))
    log_gate = (-u).astype(np.float32)
    n = rng.standard_normal((B, T, H))
    beta = (1.0 / (1.0 + np.exp(-w.beta_sigma * n))).astype(np.float32)
    if w.h0_sigma > 0:
        h0 = (w.h0_sigma * rng.standard_normal((B, H, w.d_k, w.d_v))).astype(np.float32)
    else:
        h0 = np.zeros((B, H, w.d_k, w.d_v), dtype=np.float32)
    if w.qk_spread > 0:
        mq = rng.standard_normal((B, T, H, 1))
        mk = rng.standard_normal((B, T, H, 1))
        q = (q * np.exp(w.qk_spread * mq)).astype(np.float32)
        k = (k * np.exp(w.qk_spread * mk)).astype(np.float32)
    if w.qkv_dtype == "bf16":
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    elif w.qkv_dtype != "f32":
        raise ValueError(f"unknown qkv dtype {w.qkv_dtype!r}")
    return {"q": q, "k": k, "v": v, "log_gate": log_gate, "beta": beta, "h0": h0}
