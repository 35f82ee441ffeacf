"""Pins of the CPU oracle against things other than itself (CPU only).

The pages print no worked numerical example of the layer, so the oracle is
pinned by: explicit transition products (brute force), a worked example
derived by hand from the token-wise update, closed forms of special cases,
and invariants.  Planted-mistake variants of the recurrence show that these
pins reject the plausible slips (read-before-write, dropped decay, transposed
state, wrong residual sign, dropped beta).

Pages: "SANA-WM: Efficient Minute-Scale World Modeling with Hybrid Linear
Diffusion Transformer" (summary), section 3.2: token-wise update, frame-wise
update, "Algebraic Stabilization for Spatial Token Explosion",
"Bidirectional and Chunk-Causal GDN Variants".
"""
from fractions import Fraction as Fr

import numpy as np
import pytest

from gdn_inputs import WORKLOADS, make_inputs
from oracle import bruteforce
from oracle import gdn_oracle as O

TINY = WORKLOADS[0]


def tiny(seed=0, **kw):
    w = TINY.resized(**kw) if kw else TINY
    return w, make_inputs(w, seed)


def args(x):
    return x["q"], x["k"], x["v"], x["log_gate"], x["beta"]


def rel(a, b):
    return np.max(np.abs(a - b)) / max(np.sqrt(np.mean(b * b)), 1e-300)


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("nonzero_h0", [False, True])
def test_fwd_matches_explicit_products(nonzero_h0):
    """Outputs and final state equal the explicit-product form (tiny workload)."""
    w, x = tiny()
    h0 = 0.1 * np.random.default_rng(5).standard_normal(x["h0"].shape) if nonzero_h0 else None
    o, H = O.fwd(*args(x), h0)
    ob, Hb = bruteforce.scan(*args(x), h0)
    assert rel(o, ob) < 1e-12 and rel(H, Hb) < 1e-12


def test_bwd_matches_explicit_products_of_reversed_sequence():
    """The reversed scan is the explicit-product form over the reversed tokens."""
    w, x = tiny(seed=3)
    o, H = O.bwd(*args(x))
    flip = lambda a: np.flip(a, axis=1)
    ob, Hb = bruteforce.scan(*[flip(a) for a in args(x)])
    assert rel(o, flip(ob)) < 1e-12 and rel(H, Hb) < 1e-12


def test_bidir_is_sum_of_scans_and_reports_forward_state():
    w, x = tiny(seed=4)
    h0 = 0.1 * np.random.default_rng(1).standard_normal(x["h0"].shape)
    ob, Hb = O.bidir(*args(x), h0)
    f = bruteforce.scan(*args(x), h0)
    flip = lambda a: np.flip(a, axis=1)
    r = bruteforce.scan(*[flip(a) for a in args(x)])
    assert rel(ob, f[0] + flip(r[0])) < 1e-12
    assert rel(Hb, f[1]) < 1e-12


def test_key_scale_is_applied_to_keys_only():
    w, x = tiny(seed=6)
    s = 0.25
    o, H = O.fwd(*args(x), None, key_scale=s)
    x2 = dict(x, k=x["k"] * s)
    ob, Hb = bruteforce.scan(*args(x2))
    assert rel(o, ob) < 1e-12 and rel(H, Hb) < 1e-12


# ------------------------------------------------------- worked example by hand

def _worked_inputs():
    """Three tokens, d_k = d_v = 2, H0 = I; gates chosen so all values are rational."""
    q = np.array([[0, 1], [1, 1], [1, 0]], float)
    k = np.array([[1, 0], [0, 1], [0.6, 0.8]], float)
    v = np.array([[1, 2], [3, -1], [0, 0]], float)
    g = np.log([0.5, 1.0, 0.25])
    beta = np.array([0.5, 1.0, 1.0])
    sh = lambda a: a[None, :, None]
    return (sh(q), sh(k), sh(v), g[None, :, None], beta[None, :, None]), np.eye(2)[None, None]


# Derivation (stored orientation, o = H^T q):
#  t1: H = I/2; pred = H^T k1 = (1/2, 0); e = (1/2, 2); H += (1/2) k1 e^T
#      -> H1 = [[3/4, 1], [0, 1/2]];            o1 = row 1 of H1 = (0, 1/2)
#  t2: gamma = 1; pred = row 1 of H1 = (0, 1/2); e = (3, -3/2); H += k2 e^T
#      -> H2 = [[3/4, 1], [3, -1]];             o2 = row0 + row1 = (15/4, 0)
#  t3: H = H2/4; pred = H^T (3/5, 4/5) = (57/80, -1/20); e = -pred; H += k3 e^T
#      -> H3 = [[-6/25, 7/25], [9/50, -21/100]]; o3 = row 0 = (-6/25, 7/25)
#      (check: H3^T k3 = 0 = v3, exact recall with beta = 1)
WORKED_O = [[Fr(0), Fr(1, 2)], [Fr(15, 4), Fr(0)], [Fr(-6, 25), Fr(7, 25)]]
WORKED_H = [[Fr(-6, 25), Fr(7, 25)], [Fr(9, 50), Fr(-21, 100)]]


def test_worked_example_by_hand():
    a, h0 = _worked_inputs()
    o, H = O.fwd(*a, h0)
    np.testing.assert_allclose(o[0, :, 0], np.array(WORKED_O, float), atol=1e-14)
    np.testing.assert_allclose(H[0, 0], np.array(WORKED_H, float), atol=1e-14)


# ------------------------------------------------------------ special cases

def test_P1_beta_zero_is_pure_decay():
    """beta = 0: H_T = exp(sum g) H0 and o_t = exp(Gamma_t) H0^T q_t (Gamma: global cumsum)."""
    w, x = tiny(seed=1)
    h0 = 0.1 * np.random.default_rng(2).standard_normal(x["h0"].shape)
    x = dict(x, beta=np.zeros_like(x["beta"]))
    o, H = O.fwd(*args(x), h0)
    Gam = np.cumsum(x["log_gate"].astype(np.float64), axis=1)   # [B,T,H]
    exp_o = np.exp(Gam)[..., None] * np.einsum("bthi,bhij->bthj", x["q"].astype(np.float64), h0)
    assert rel(o, exp_o) < 1e-13
    assert rel(H, np.exp(Gam[:, -1])[:, :, None, None] * h0) < 1e-13


def _orthonormal_frames(F, d, rng):
    return np.concatenate([np.linalg.qr(rng.standard_normal((d, d)))[0].T for _ in range(F)])


def test_P2_exact_recall_with_orthonormal_keys():
    """gamma = 1, beta = 1, each frame's keys an orthonormal basis (S = d_k = 16).

    After each frame H = K_f^T V_f (exact recall k_j^T H = v_j); mid-frame
    H_t = H0 - sum_{i<=t} k_i k_i^T H0 + sum_{i<=t} k_i v_i^T.
    """
    rng = np.random.default_rng(11)
    F, d = 3, 16
    K = _orthonormal_frames(F, d, rng)
    V = rng.standard_normal((F * d, d))
    Q = rng.standard_normal((F * d, d))
    sh = lambda a: a[None, :, None]
    g = np.zeros((1, F * d, 1))
    b = np.ones((1, F * d, 1))
    h0 = rng.standard_normal((1, 1, d, d))
    o, H = O.fwd(sh(Q), sh(K), sh(V), g, b, h0)
    Kf, Vf = K[-d:], V[-d:]
    np.testing.assert_allclose(H[0, 0], Kf.T @ Vf, atol=1e-12)
    np.testing.assert_allclose(Kf @ H[0, 0], Vf, atol=1e-12)
    # mid-frame closed form in frame 0, token t = 6
    t = 6
    Kt, Vt = K[: t + 1], V[: t + 1]
    Ht = h0[0, 0] - Kt.T @ (Kt @ h0[0, 0]) + Kt.T @ Vt
    np.testing.assert_allclose(o[0, t, 0], Ht.T @ Q[t], atol=1e-12)
    # Reading B reaches the same state at frame ends here
    _, Hj = O.jacobi(sh(Q), sh(K), sh(V), g, b, h0, tokens_per_frame=d)
    np.testing.assert_allclose(Hj[0, 0], Kf.T @ Vf, atol=1e-12)


def test_P3_single_token_frames_jacobi_equals_tokenwise():
    w, x = tiny(seed=2)
    h0 = 0.1 * np.random.default_rng(3).standard_normal(x["h0"].shape)
    o, H = O.fwd(*args(x), h0)
    oj, Hj = O.jacobi(*args(x), h0, tokens_per_frame=1)
    assert rel(oj, o) < 1e-12 and rel(Hj, H) < 1e-12


def test_P4_orthonormal_keys_gate_on_first_token_states_agree():
    """Orthonormal keys per frame, gate only on each frame's first token: the
    frame-level (Reading B) and token-wise (Reading A) end states coincide."""
    rng = np.random.default_rng(13)
    F, d = 3, 16
    K = _orthonormal_frames(F, d, rng)
    V, Q = rng.standard_normal((F * d, d)), rng.standard_normal((F * d, d))
    g = np.zeros(F * d)
    g[::d] = -rng.uniform(0.1, 0.5, F)
    beta = rng.uniform(0, 1, F * d)
    sh = lambda a: a[None, :, None]
    h0 = rng.standard_normal((1, 1, d, d))
    _, H = O.fwd(sh(Q), sh(K), sh(V), sh(g), sh(beta), h0)
    _, Hj = O.jacobi(sh(Q), sh(K), sh(V), sh(g), sh(beta), h0, tokens_per_frame=d)
    np.testing.assert_allclose(Hj, H, atol=1e-12)


def test_P3b_single_token_frames_reversed_and_bidirectional_jacobi_equal_tokenwise():
    """One token per frame: the reversed and bidirectional frame-level scans
    are the token-wise ones (which the explicit-product pins fix)."""
    w, x = tiny(seed=4)
    h0 = 0.1 * np.random.default_rng(6).standard_normal(x["h0"].shape)
    for jf, tf in ((O.jacobi_bwd, O.bwd), (O.jacobi_bidir, O.bidir)):
        o, H = tf(*args(x), h0)
        oj, Hj = jf(*args(x), h0, tokens_per_frame=1)
        assert rel(oj, o) < 1e-12 and rel(Hj, H) < 1e-12


def test_P4b_reversed_jacobi_takes_the_gate_of_the_frame_last_token():
    """Orthonormal keys per frame, gate only on each frame's last token: the
    reversed frame-level scan and the reversed token-wise scan reach the same
    state (the reversed scan meets that token first)."""
    rng = np.random.default_rng(14)
    F, d = 3, 16
    K = _orthonormal_frames(F, d, rng)
    V, Q = rng.standard_normal((F * d, d)), rng.standard_normal((F * d, d))
    g = np.zeros(F * d)
    g[d - 1::d] = -rng.uniform(0.1, 0.5, F)
    beta = rng.uniform(0, 1, F * d)
    sh = lambda a: a[None, :, None]
    h0 = rng.standard_normal((1, 1, d, d))
    _, H = O.bwd(sh(Q), sh(K), sh(V), sh(g), sh(beta), h0)
    _, Hj = O.jacobi_bwd(sh(Q), sh(K), sh(V), sh(g), sh(beta), h0, tokens_per_frame=d)
    np.testing.assert_allclose(Hj, H, atol=1e-12)
    # with the gate on the first token instead, the decays land elsewhere
    g2 = np.roll(g, -(d - 1))
    _, Hj2 = O.jacobi_bwd(sh(Q), sh(K), sh(V), sh(g2), sh(beta), h0, tokens_per_frame=d)
    _, H2 = O.bwd(sh(Q), sh(K), sh(V), sh(g2), sh(beta), h0)
    assert np.max(np.abs(Hj2 - H2)) > 1e-3


def test_P6_chunk_causal_single_chunk_is_bidirectional_and_per_token_chunks_add_the_token_term():
    """One chunk spanning the sequence is the bidirectional layer; chunks of
    one single-token frame add to the forward output exactly each token's
    own reversed-scan term, the read of v beta k^T with q."""
    w, x = tiny(seed=5)
    h0 = 0.1 * np.random.default_rng(7).standard_normal(x["h0"].shape)
    o, H = O.chunk_causal(*args(x), h0, tokens_per_frame=TINY.tokens_per_frame,
                          first_chunk_frames=TINY.frames, chunk_frames=TINY.frames)
    ob, Hb = O.bidir(*args(x), h0)
    assert rel(o, ob) < 1e-12 and rel(H, Hb) < 1e-12
    q, k, v, g, b = args(x)
    o1, _ = O.chunk_causal(q, k, v, g, b, h0, tokens_per_frame=1)
    of, _ = O.fwd(q, k, v, g, b, h0)
    # a one-token reversed scan from zero: H = beta k v^T, o = H^T q = beta (q.k) v
    q64, k64, v64, b64 = (np.asarray(t, dtype=np.float64) for t in (q, k, v, b))
    own = (b64 * np.einsum("bthi,bthi->bth", q64, k64))[..., None] * v64
    assert rel(o1, of + own) < 1e-12


def test_P7_chunk_causal_outputs_do_not_depend_on_later_chunks():
    """Causality at chunk granularity: changing the inputs of the last chunk
    leaves every earlier chunk's outputs unchanged, and changes the last
    chunk's."""
    w, x = tiny(seed=6, frames=5, tokens_per_frame=4)
    S = 4
    kw = dict(tokens_per_frame=S, first_chunk_frames=2, chunk_frames=2)   # chunks 2, 2, 1
    o, _ = O.chunk_causal(*args(x), **kw)
    y = {n: np.array(x[n], copy=True) for n in x}
    y["v"][:, 4 * S:] += 1.0
    y["k"][:, 4 * S:] *= -1.0
    o2, _ = O.chunk_causal(*args(y), **kw)
    assert np.array_equal(o[:, :4 * S], o2[:, :4 * S])
    assert np.max(np.abs(o[:, 4 * S:] - o2[:, 4 * S:])) > 1e-3
    # the bidirectional layer is not causal: the same change reaches the first chunk
    ob, _ = O.bidir(*args(x))
    ob2, _ = O.bidir(*args(y))
    assert np.max(np.abs(ob[:, :2 * S] - ob2[:, :2 * S])) > 1e-6
    assert O.chunk_bounds(5, 2, 2) == [(0, 2), (2, 4), (4, 5)]
    assert O.chunk_bounds(121, 4, 3)[:3] == [(0, 4), (4, 7), (7, 10)] and O.chunk_bounds(121, 4, 3)[-1] == (118, 121)


def test_P5_same_key_twice_overwrites():
    rng = np.random.default_rng(17)
    d = 8
    kk = rng.standard_normal(d)
    kk /= np.linalg.norm(kk)
    K = np.stack([kk, kk])
    V = rng.standard_normal((2, d))
    sh = lambda a: a[None, :, None]
    _, H = O.fwd(sh(rng.standard_normal((2, d))), sh(K), sh(V), np.zeros((1, 2, 1)),
                 np.ones((1, 2, 1)), rng.standard_normal((1, 1, d, d)))
    np.testing.assert_allclose(kk @ H[0, 0], V[1], atol=1e-12)


# -------------------------------------------------------------- invariants

def test_I1_linear_in_values_and_initial_state():
    w, x = tiny(seed=7)
    rng = np.random.default_rng(8)
    v2, h1, h2 = rng.standard_normal(x["v"].shape), rng.standard_normal(x["h0"].shape), \
        rng.standard_normal(x["h0"].shape)
    a, b = 0.7, -1.3
    q, k, v, g, be = args(x)
    v = v.astype(np.float64)
    o1, H1 = O.fwd(q, k, v, g, be, h1)
    o2, H2 = O.fwd(q, k, v2, g, be, h2)
    o3, H3 = O.fwd(q, k, a * v + b * v2, g, be, a * h1 + b * h2)
    assert rel(o3, a * o1 + b * o2) < 1e-12 and rel(H3, a * H1 + b * H2) < 1e-12


def test_I2_chunk_invariance_steps_and_half_frames():
    """FWD over all frames == chained one-frame steps == chained half-frame pieces."""
    w, x = tiny(seed=9)
    h0 = 0.1 * np.random.default_rng(4).standard_normal(x["h0"].shape)
    o, H = O.fwd(*args(x), h0)
    for piece in (w.tokens_per_frame, w.tokens_per_frame // 2, 5):
        s, outs = h0, []
        for t0 in range(0, w.tokens, piece):
            sl = slice(t0, t0 + piece)
            oo, s = O.step(*[a[:, sl] for a in args(x)], s)
            outs.append(oo)
        assert rel(np.concatenate(outs, axis=1), o) < 1e-13 and rel(s, H) < 1e-13


def test_I4_head_and_batch_permutation_equivariance():
    w, x = tiny(seed=10, batch=2, heads=3)
    h0 = 0.1 * np.random.default_rng(4).standard_normal(x["h0"].shape)
    o, H = O.bidir(*args(x), h0)
    ph, pb = np.array([2, 0, 1]), np.array([1, 0])
    perm = lambda a: a[pb][:, :, ph] if a.ndim >= 3 and a.shape[2] == 3 else a
    xp = {n: x[n][pb][:, :, ph] for n in ("q", "k", "v", "log_gate", "beta")}
    op, Hp = O.bidir(*args(xp), h0[pb][:, ph])
    assert rel(op, o[pb][:, :, ph]) < 1e-13 and rel(Hp, H[pb][:, ph]) < 1e-13


def test_I5_non_expansive_bound():
    """On the documented domain (g <= 0, beta in [0,1], |k| <= 1) the state obeys
    |H_T|_F <= |H_0|_F + sum_t beta_t |k_t| |v_t|."""
    w, x = tiny(seed=12)
    h0 = np.random.default_rng(3).standard_normal(x["h0"].shape)
    _, H = O.fwd(*args(x), h0)
    k64, v64 = x["k"].astype(float), x["v"].astype(float)
    bound = np.linalg.norm(h0[0, 0]) + np.sum(
        x["beta"][0, :, 0] * np.linalg.norm(k64[0, :, 0], axis=-1) * np.linalg.norm(v64[0, :, 0], axis=-1))
    assert np.linalg.norm(H[0, 0]) <= bound


def test_I6_spatial_key_scale_keeps_frame_transition_non_expansive():
    """Algebraic Stabilization: with unit keys scaled by 1/sqrt(S) and beta <= 1,
    |I - K^T diag(beta) K|_2 <= 1.  The exact condition is lambda_max <= 2; without
    the scale, S = 880 unit keys at d = 112 break it."""
    rng = np.random.default_rng(0)
    S, d = 880, 112
    K = rng.standard_normal((S, d))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    beta = 1 / (1 + np.exp(-rng.standard_normal(S)))
    for scale, ok in ((1 / np.sqrt(S), True), (1.0, False)):
        Ks = K * scale
        M = np.eye(d) - Ks.T @ (beta[:, None] * Ks)
        assert (np.linalg.norm(M, 2) <= 1 + 1e-12) == ok


def test_I8_resume_is_bit_identical():
    w, x = tiny(seed=14)
    h0 = 0.1 * np.random.default_rng(4).standard_normal(x["h0"].shape)
    S = w.tokens_per_frame
    s, outs = h0, []
    for f in range(w.frames):
        oo, s = O.step(*[a[:, f * S:(f + 1) * S] for a in args(x)], s)
        outs.append(oo)
    saved = s.copy()
    # stop after frame 1, save, reload, continue
    s2 = h0
    for f in range(2):
        _, s2 = O.step(*[a[:, f * S:(f + 1) * S] for a in args(x)], s2)
    reloaded = np.array(s2.tolist())
    o_last, s3 = O.step(*[a[:, 2 * S:] for a in args(x)], reloaded)
    assert np.array_equal(s3, saved) and np.array_equal(o_last, outs[2])


# ----------------------------------------------------- planted mistakes

def _mutant_fwd(kind, q, k, v, g, beta, h0):
    """Token recurrence with one planted slip (CPU only); single (batch, head)."""
    H = h0.copy()
    out = []
    for t in range(len(q)):
        prev = H.copy()
        if kind != "no_decay":
            H = np.exp(g[t]) * H
        src = prev if kind == "predict_before_decay" else H
        pred = src.T @ k[t]
        e = (pred - v[t]) if kind == "wrong_sign" else (v[t] - pred)
        b = 1.0 if kind == "no_beta" else beta[t]
        newH = H + b * np.outer(k[t], e)
        if kind == "read_before_write":
            out.append(H.T @ q[t])
        elif kind == "transposed_read":
            out.append(newH @ q[t])
        else:
            out.append(newH.T @ q[t])
        H = newH
    return np.array(out), H


MUTANTS = ["no_decay", "predict_before_decay", "wrong_sign", "no_beta",
           "read_before_write", "transposed_read"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_reject_planted_mistakes(kind):
    """Each slip fails the worked example or the brute-force pin."""
    a, h0 = _worked_inputs()
    sq = lambda z: z[0, :, 0]
    o_m, H_m = _mutant_fwd(kind, *[sq(z) for z in a], h0[0, 0])
    worked_ok = (np.allclose(o_m, np.array(WORKED_O, float), atol=1e-12)
                 and np.allclose(H_m, np.array(WORKED_H, float), atol=1e-12))
    w, x = tiny(seed=0)
    hh = 0.1 * np.random.default_rng(5).standard_normal(x["h0"].shape)
    ob, Hb = bruteforce.scan(*args(x), hh)
    o_m2, H_m2 = _mutant_fwd(kind, *[sq(z).astype(float) for z in args(x)], hh[0, 0])
    brute_ok = rel(o_m2, ob[0, :, 0]) < 1e-9 and rel(H_m2, Hb[0, 0]) < 1e-9
    assert not (worked_ok and brute_ok)
    # and the unmutated recurrence passes both
    o_r, H_r = _mutant_fwd("none", *[sq(z) for z in a], h0[0, 0])
    assert np.allclose(o_r, np.array(WORKED_O, float), atol=1e-12)


# ----------------------------------------------------- feature prologue (keys and queries)
# [WM-summary] section 3.2, "Algebraic Stabilization for Spatial Token Explosion":
# key features ReLU(RMSNorm(K)) with squared norm about d_k, then 1/sqrt(D*S).

def _key_pins(kf):
    """The key-feature pins, as a predicate on a candidate implementation."""
    ok = True
    # worked by hand: k = (3, -4, 0, 0): mean square 25/4, RMS 5/2
    ok &= np.allclose(kf(np.array([3.0, -4.0, 0.0, 0.0]), 0.0), [1.2, 0.0, 0.0, 0.0], rtol=0, atol=1e-15)
    ok &= np.allclose(kf(np.array([3.0, -4.0, 0.0, 0.0]), 1e-6), [3 / np.sqrt(6.25 + 1e-6), 0, 0, 0],
                      rtol=0, atol=1e-15)
    rng = np.random.default_rng(21)
    k = rng.standard_normal((5, 7, 3, 112)) * np.exp(rng.standard_normal((5, 7, 3, 1)))
    # a non-negative key keeps all of its energy: squared norm exactly d_k
    ok &= np.allclose(np.sum(kf(np.abs(k), 0.0) ** 2, axis=-1), 112.0, rtol=1e-13, atol=0)
    # ReLU splits a key's normalised components between k and -k
    both = kf(k, 0.0) + kf(-k, 0.0)
    ok &= np.allclose(both, np.abs(k) / np.sqrt(np.mean(k * k, axis=-1, keepdims=True)), rtol=1e-13, atol=0)
    # scale invariance per token
    ok &= np.allclose(kf(k * 7.5, 0.0), kf(k, 0.0), rtol=1e-13, atol=1e-15)
    return bool(ok)


def _query_pins(qf):
    ok = True
    ok &= np.allclose(qf(np.array([3.0, 4.0]), 0.0), [0.6, 0.8], rtol=0, atol=1e-15)
    rng = np.random.default_rng(22)
    q = rng.standard_normal((4, 5, 3, 64)) * np.exp(rng.standard_normal((4, 5, 3, 1)))
    ok &= np.allclose(np.sum(qf(q, 0.0) ** 2, axis=-1), 1.0, rtol=1e-13, atol=0)
    ok &= np.allclose(qf(-q, 0.0), -qf(q, 0.0), rtol=0, atol=0)          # odd: no ReLU on queries
    ok &= np.allclose(qf(q * 0.03, 0.0), qf(q, 0.0), rtol=1e-13, atol=1e-15)
    return bool(ok)


def test_P8_key_features_by_hand_and_invariants():
    assert _key_pins(O.key_features)
    # zero key: zeros (eps keeps the division finite); NaN stays NaN
    assert np.array_equal(O.key_features(np.zeros(16)), np.zeros(16))
    assert np.all(np.isnan(O.key_features(np.array([1.0, np.nan, -2.0, 3.0]))))


def test_P8_query_normalisation_by_hand_and_invariants():
    assert _query_pins(O.query_features)
    assert np.array_equal(O.query_features(np.zeros(16)), np.zeros(16))
    # the default epsilon enters the sum of squares
    assert np.isclose(O.query_features(np.array([1e-3, 0.0]))[0], 1e-3 / np.sqrt(1e-6 + 1e-6), rtol=1e-15)


def test_P8_spatial_scale_bounds_the_frame_trace_by_one():
    """Page claim: with RMS-normalised ReLU keys, beta <= 1 and the scale
    1/sqrt(D*S), tr(K^T diag(beta) K) <= 1, so |I - K^T diag(beta) K|_2 <= 1;
    the 1/sqrt(D) scale alone breaks it at S = 880."""
    rng = np.random.default_rng(23)
    S, d = 880, 112
    raw = rng.standard_normal((S, d)) * np.exp(rng.standard_normal((S, 1)))
    beta = 1 / (1 + np.exp(-2 * rng.standard_normal(S)))
    kb = O.key_features(raw)
    for scale, ok in ((1 / np.sqrt(d * S), True), (1 / np.sqrt(d), False)):
        Ks = kb * scale
        A = Ks.T @ (beta[:, None] * Ks)
        assert (np.trace(A) <= 1.0) == ok
        assert (np.linalg.norm(np.eye(d) - A, 2) <= 1 + 1e-12) == ok


PROLOGUE_MUTANTS = {
    "sum_not_mean": (lambda k, e: np.maximum(k / np.sqrt(np.sum(k * k, -1, keepdims=True) + e), 0), None),
    "relu_before_norm": (lambda k, e: (lambda r: r / np.sqrt(np.mean(r * r, -1, keepdims=True) + e))(
        np.maximum(k, 0)), None),
    "no_relu": (lambda k, e: k / np.sqrt(np.mean(k * k, -1, keepdims=True) + e), None),
    "abs_not_relu": (lambda k, e: np.abs(k) / np.sqrt(np.mean(k * k, -1, keepdims=True) + e), None),
    "query_rms": (None, lambda q, e: q / np.sqrt(np.mean(q * q, -1, keepdims=True) + e)),
    "query_relu": (None, lambda q, e: np.maximum(q / np.sqrt(np.sum(q * q, -1, keepdims=True) + e), 0)),
    "query_unnormalised": (None, lambda q, e: q),
}


@pytest.mark.parametrize("kind", list(PROLOGUE_MUTANTS))
def test_prologue_pins_reject_planted_mistakes(kind):
    kf, qf = PROLOGUE_MUTANTS[kind]
    if kf is not None:
        assert not _key_pins(kf)
    if qf is not None:
        assert not _query_pins(qf)
