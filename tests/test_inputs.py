"""The seeded input generator: determinism, shapes, distributions, bf16 rounding (CPU)."""
import numpy as np
import pytest
import torch

from gdn_inputs import WORKLOADS, bf16_round, make_inputs


def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0, -0.0], np.float32)])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(bf16_round(x), ref)


@pytest.mark.parametrize("i", [0, 1])
def test_deterministic_and_shaped(i):
    w = WORKLOADS[i].resized(frames=2) if i else WORKLOADS[i]
    a, b = make_inputs(w, 3), make_inputs(w, 3)
    for n in a:
        assert np.array_equal(a[n], b[n]) and a[n].dtype == np.float32
    B, T, H = w.batch, w.tokens, w.heads
    assert a["q"].shape == (B, T, H, w.d_k) and a["v"].shape == (B, T, H, w.d_v)
    assert a["log_gate"].shape == (B, T, H) and a["h0"].shape == (B, H, w.d_k, w.d_v)
    assert not np.array_equal(make_inputs(w, 4)["q"], a["q"])


def test_distributions():
    w = WORKLOADS[4].resized(frames=3, tokens_per_frame=40, heads=5)
    x = make_inputs(w, 0)
    assert np.allclose(np.linalg.norm(x["k"], axis=-1), 1, atol=2 ** -7)
    assert np.array_equal(bf16_round(x["v"]), x["v"])
    g = x["log_gate"]
    assert (g <= -w.gate_lo).all() and (g >= -w.gate_hi).all()
    # frame-shared gates in this workload
    gf = g.reshape(w.batch, w.frames, w.tokens_per_frame, w.heads)
    assert (gf == gf[:, :, :1]).all()
    assert ((x["beta"] > 0) & (x["beta"] < 1)).all()
    assert 0.05 < x["h0"].std() < 0.15
    assert (make_inputs(WORKLOADS[0], 0)["h0"] == 0).all()


def test_raw_projections_for_the_feature_prologue():
    """qk_spread > 0: q, k are left unnormalised with token magnitudes spread
    over about a decade; the other tensors are drawn exactly as without it."""
    w = WORKLOADS[2].resized(frames=2, tokens_per_frame=50, heads=3)
    a, b = make_inputs(w, 5), make_inputs(w.resized(qk_spread=1.0), 5)
    for n in ("v", "log_gate", "beta", "h0"):
        assert np.array_equal(a[n], b[n])
    nk = np.linalg.norm(b["k"].astype(np.float64), axis=-1)
    assert nk.max() / nk.min() > 10 and np.array_equal(bf16_round(b["k"]), b["k"])
    assert not np.allclose(np.linalg.norm(b["q"], axis=-1), 1, atol=0.1)
