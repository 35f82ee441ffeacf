"""The chunked decomposition the GPU kernels use reproduces the oracle in
float64 (CPU).  This pins the kernels' algebra (sub-chunk WY/UT form, segment
maps, segment chain, reversed traversal with ragged pieces), not the oracle."""
import numpy as np
import pytest

from gdn_inputs import WORKLOADS, make_inputs
from oracle import gdn_oracle as O
from tests import chunk_model as M


def rel(a, b):
    return np.max(np.abs(a - b)) / np.sqrt(np.mean(b * b))


@pytest.mark.parametrize("direction", ["fwd", "bwd", "bidir"])
@pytest.mark.parametrize("T,L", [(300, 128), (300, 64), (257, 192), (64, 64), (5, 64)])
def test_chunked_model_matches_oracle(direction, T, L):
    w = WORKLOADS[4].resized(frames=1, tokens_per_frame=T, heads=2, d_k=32, d_v=48)
    x = make_inputs(w, 1)
    a = (x["q"], x["k"], x["v"], x["log_gate"], x["beta"])
    ro, rH = O.forward(direction, *a, x["h0"], key_scale=0.7)
    mo, mH = M.forward(direction, *a, x["h0"], key_scale=0.7, L=L)
    assert rel(mo, ro) < 1e-11 and rel(mH, rH) < 1e-11


def test_segment_map_is_affine_state_map():
    rng = np.random.default_rng(0)
    n, dk, dv = 150, 16, 24
    K = rng.standard_normal((n, dk)) / 4
    V = rng.standard_normal((n, dv))
    g = -rng.uniform(0.01, 0.2, n)
    b = rng.uniform(0, 1, n)
    pieces = [np.arange(a, min(a + 64, n)) for a in range(0, n, 64)]
    P, Qm = M.segment_map(K, V, g, b, pieces)
    H0 = rng.standard_normal((dk, dv))
    H = H0
    for idx in pieces:
        _, H = M.chunk_step(H, np.zeros((len(idx), dk)), K[idx], V[idx], g[idx], b[idx])
    assert np.allclose(P @ H0 + Qm, H, atol=1e-12)


def test_blocked_inverse_and_r_form_match_wy_form():
    """The blocked triangular inverse equals (I + A)^-1, and the R form of V'
    equals the WY/UT form U - W H."""
    rng = np.random.default_rng(5)
    n, d = 64, 24
    K = rng.standard_normal((n, d))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    V = rng.standard_normal((n, d))
    g = -rng.uniform(0.001, 0.1, n)
    beta = 1 / (1 + np.exp(-rng.standard_normal(n)))
    H = rng.standard_normal((d, d))
    G, E, W, U = M.wy(K, V, g, beta)
    A = np.tril((beta[:, None] * (K @ K.T)) * E, -1)
    Tm = M.blocked_inverse(A)
    assert np.max(np.abs(Tm - np.linalg.inv(np.eye(n) + A))) < 1e-12
    R = V - np.exp(G)[:, None] * (K @ H)
    assert np.max(np.abs(Tm @ (beta[:, None] * R) - (U - W @ H))) < 1e-11
