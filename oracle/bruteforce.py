"""Brute-force form of the gated delta rule: explicit transition products.

TEST INFRASTRUCTURE ONLY (imported by ``tests/`` to pin the oracle).

Unrolling the token-wise update of [WM-summary] ("SANA-WM: Efficient
Minute-Scale World Modeling with Hybrid Linear Diffusion Transformer",
section 3.2, "Frame-wise Gated DeltaNet (GDN)", token-wise update) gives, in
the stored orientation H = S^T,
    H_t = Phi_t H_{t-1} + beta_t k_t v_t^T,  Phi_t = gamma_t (I - beta_t k_t k_t^T)
so that, with no loop-carried state across tokens,
    H_t = (Phi_t ... Phi_1) H_0 + sum_{i<=t} (Phi_t ... Phi_{i+1}) beta_i k_i v_i^T
    o_t = H_t^T q_t.
Every H_t is formed from scratch out of explicit d_k x d_k matrices: O(T^2 d^3)
work, for tiny inputs only.  It shares no code with ``gdn_oracle``.
"""
from __future__ import annotations

import numpy as np


def transition(g, beta, k):
    """Phi = exp(g) (I - beta k k^T) as an explicit d_k x d_k matrix."""
    k = np.asarray(k, dtype=np.float64)
    return np.exp(float(g)) * (np.eye(k.shape[0]) - float(beta) * np.outer(k, k))


def state_at(t, q, k, v, g, beta, h0):
    """H_t for one (batch, head): q,k [T,d_k], v [T,d_v], g, beta [T]."""
    dk, dv = k.shape[1], v.shape[1]
    acc = np.zeros((dk, dv))
    R = np.eye(dk)                                   # Phi_t ... Phi_{i+1}
    for i in range(t, -1, -1):
        acc += R @ (float(beta[i]) * np.outer(k[i], v[i]))
        R = R @ transition(g[i], beta[i], k[i])
    return acc + R @ np.asarray(h0, dtype=np.float64)


def scan(q, k, v, log_gate, beta, h0=None, key_scale=1.0):
    """Outputs and final state of the forward scan, all by explicit products.

    Layouts as the oracle: q,k [B,T,H,d_k], v [B,T,H,d_v], gates [B,T,H].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64) * float(key_scale)
    v = np.asarray(v, dtype=np.float64)
    B, T, Hh, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, Hh, dv))
    Hs = np.zeros((B, Hh, dk, dv))
    for b in range(B):
        for h in range(Hh):
            H0 = np.zeros((dk, dv)) if h0 is None else np.asarray(h0, np.float64)[b, h]
            args = (q[b, :, h], k[b, :, h], v[b, :, h], log_gate[b, :, h], beta[b, :, h])
            for t in range(T):
                Ht = state_at(t, *args, H0)
                o[b, t, h] = Ht.T @ q[b, t, h]
                if t == T - 1:
                    Hs[b, h] = Ht
    return o, Hs
