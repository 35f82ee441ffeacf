"""GPU parity: libgdn (through the C ABI) against the float64 oracle.

Every case runs on seeded synthetic inputs from ``gdn_inputs`` with the
workloads' distributions, at sizes the oracle finishes in seconds that still
span several 64-token chunks and a ragged tail.  The full-size workloads are
checked on sampled heads (heads are independent, so a head's whole output
sequence and final state are exact oracle targets).
"""
import numpy as np
import pytest

from gdn_inputs import WORKLOADS, make_inputs
from oracle import gdn_oracle as O
from tests.gpu_util import TOL, oracle_args, rel_err, to_device, to_numpy

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

G = None


def setup_module():
    global G
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_frame_amd as lib
    G = lib
    G.lib()


def run_gpu(w, x, direction, algo, out_dtype=None):
    d = to_device(x, w.qkv_dtype)
    h0 = d["h0"] if np.any(x["h0"]) else None
    out, hT = G.forward(d["q"], d["k"], d["v"], d["log_gate"], d["beta"], h0, direction,
                        tokens_per_frame=w.tokens_per_frame, algo=algo, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return to_numpy(out), to_numpy(hT)


def check(w, x, direction, algo, heads=None, out_dtype=None):
    o, hT = run_gpu(w, x, direction, algo, out_dtype)
    a, h0 = oracle_args(x, heads)
    ro, rH = O.forward(direction, *a, h0)
    if heads is not None:
        o, hT = o[:, :, heads], hT[:, heads]
    eo, eh = rel_err(o, ro), rel_err(hT, rH)
    print(f"[parity] {w.name} {direction} {algo}: out {eo:.3e} state {eh:.3e}", flush=True)
    tol = TOL[w.qkv_dtype]
    assert eo <= tol and eh <= tol, (eo, eh)
    return eo, eh


ALGOS = ["recurrent", "chunked"]


def need(algo, w):
    if algo == "chunked" and w.qkv_dtype != "bf16":
        pytest.skip("the chunked path takes bf16 q/k/v")


@pytest.mark.parametrize("direction", ["fwd", "bwd", "bidir"])
def test_tiny_fp32(direction):
    """Tiny workload (3 frames x 16 tokens, d = 16, fp32): fp32 bar 1e-4."""
    w = WORKLOADS[0]
    x = make_inputs(w, 0)
    check(w, x, direction, "auto", out_dtype=torch.float32)


@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_tiny_fp32_nonzero_initial_state(direction):
    w = WORKLOADS[0].resized(h0_sigma=0.1)
    x = make_inputs(w, 1)
    check(w, x, direction, "recurrent", out_dtype=torch.float32)


SMALL = {
    "clip5s": WORKLOADS[1].resized(frames=3, heads=2),
    "clip60s": WORKLOADS[2].resized(frames=2, heads=3),
    "stream": WORKLOADS[3].resized(frames=3, heads=2),
    "batched": WORKLOADS[4].resized(frames=3, heads=3),
    "ragged": WORKLOADS[1].resized(frames=2, tokens_per_frame=201, heads=2),
    "short": WORKLOADS[4].resized(frames=1, tokens_per_frame=5, heads=2, h0_sigma=0.3),
}


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("direction", ["fwd", "bwd", "bidir"])
def test_small_bf16(algo, name, direction):
    w = SMALL[name]
    need(algo, w)
    check(w, make_inputs(w, 0), direction, algo)


@pytest.mark.parametrize("algo", ALGOS)
def test_bf16_output(algo):
    """A bf16 output is the fp32 result rounded once: the bar widens by the
    rounding of the largest element, 2^-8 max|ref| / RMS(ref)."""
    w = SMALL["batched"]
    need(algo, w)
    x = make_inputs(w, 2)
    o, hT = run_gpu(w, x, "bidir", algo, out_dtype=torch.bfloat16)
    ro, rH = O.bidir(*oracle_args(x)[0], x["h0"])
    rms = np.sqrt(np.mean(ro * ro))
    bound = TOL["bf16"] + 2.0 ** -8 * np.max(np.abs(ro)) / rms
    assert rel_err(o, ro) <= bound and rel_err(hT, rH) <= TOL["bf16"]


@pytest.mark.parametrize("direction", ["fwd", "bidir"])
@pytest.mark.parametrize("algo", ALGOS)
def test_bf16_output_is_the_fp32_output_rounded(algo, direction):
    """The bf16 output mode stores the fp32 result rounded once to the nearest
    bf16 (ties to even): element for element it equals the fp32 output of the
    same call rounded by torch, and that fp32 output meets the bar, so the
    one rounding is the mode's only departure from it."""
    w = SMALL["batched"]
    need(algo, w)
    x = make_inputs(w, 2)
    d = to_device(x, w.qkv_dtype)
    h0 = d["h0"] if np.any(x["h0"]) else None
    outs = []
    for odt in (torch.float32, torch.bfloat16):
        out, _ = G.forward(d["q"], d["k"], d["v"], d["log_gate"], d["beta"], h0, direction,
                           tokens_per_frame=w.tokens_per_frame, algo=algo, out_dtype=odt)
        outs.append(out)
    torch.cuda.synchronize()
    rounded = outs[0].to(torch.bfloat16)
    assert outs[1].dtype == torch.bfloat16
    assert torch.equal(outs[1].view(torch.int16), rounded.view(torch.int16))
    a, oh0 = oracle_args(x)
    ro, _ = O.forward(direction, *a, oh0)
    assert rel_err(to_numpy(outs[0]), ro) <= TOL[w.qkv_dtype]


@pytest.mark.parametrize("algo", ALGOS)
def test_step_chain_matches_oracle_and_forward(algo):
    """Chunk-causal streaming: chained one-frame steps, state carried (in place)."""
    w = SMALL["stream"].resized(h0_sigma=0.1)
    need(algo, w)
    x = make_inputs(w, 3)
    d = to_device(x, w.qkv_dtype)
    S = w.tokens_per_frame
    state = d["h0"].clone()
    outs = []
    for f in range(w.frames):
        sl = slice(f * S, (f + 1) * S)
        o, _ = G.step(*(d[n][:, sl].contiguous() for n in ("q", "k", "v", "log_gate", "beta")),
                      state, state, algo=algo)
        outs.append(o)
    o = to_numpy(torch.cat(outs, dim=1))
    hT = to_numpy(state)
    ro, rH = O.fwd(*oracle_args(x)[0], x["h0"])
    assert rel_err(o, ro) <= TOL["bf16"] and rel_err(hT, rH) <= TOL["bf16"]
    fo, fH = run_gpu(w, x, "fwd", algo)
    # same kernels, same inputs: the streamed and whole-sequence results agree closely
    assert rel_err(o, fo) <= 1e-2 and rel_err(hT, fH) <= 1e-2


@pytest.mark.parametrize("algo", ALGOS)
def test_chunked_matches_recurrent_gpu(algo):
    """Both GPU paths agree with each other on a multi-chunk bf16 case."""
    w = SMALL["clip60s"]
    x = make_inputs(w, 4)
    a = run_gpu(w, x, "bidir", "recurrent")
    b = run_gpu(w, x, "bidir", algo)
    assert rel_err(b[0], a[0]) <= 2e-2 and rel_err(b[1], a[1]) <= 2e-2


@pytest.mark.parametrize("name,seg", [("clip60s", 256), ("batched", 192), ("ragged", 64), ("clip5s", 1024)])
def test_concurrent_scans_match_in_order_schedule(name, seg):
    """A bidirectional chunked call gives bit-identical results whether the two
    scans overlap on the library's second stream or run in order on the
    caller's stream (same kernels, same inputs, no reduction order changes):
    7, 14, 7 and 3 segments, batch 2 with an initial state, a ragged tail."""
    w = SMALL[name]
    x = make_inputs(w, 5)
    with G.tuning(segment_tokens=seg):
        with G.tuning(serial_scans=True):
            a = run_gpu(w, x, "bidir", "chunked")
        b = run_gpu(w, x, "bidir", "chunked")
        c = run_gpu(w, x, "bidir", "chunked")
    for u, v in ((a, b), (a, c)):
        assert np.array_equal(u[0], v[0]) and np.array_equal(u[1], v[1])
    ro, rH = O.bidir(*oracle_args(x)[0], x["h0"])
    assert rel_err(b[0], ro) <= TOL["bf16"] and rel_err(b[1], rH) <= TOL["bf16"]


@pytest.mark.parametrize("prologue", [False, True])
@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_inverse_reuse_is_bit_identical(direction, prologue):
    """An output kernel that loads the segment-map kernel's sub-chunk
    inverses gives bit-identical outputs and final states to forming them
    again (the same rows and arithmetic): 1005 tokens in segments of 192 (6
    segments, a ragged last sub-chunk), d = 112, with and without the feature
    prologue; both agree with the oracle.  (Two-scan calls always form
    them.)"""
    w = WORKLOADS[1].resized(frames=5, tokens_per_frame=201, heads=2, qk_spread=1.0 if prologue else 0.0)
    x = make_inputs(w, 22)
    c = 112 ** -0.5 if prologue else 1.0

    def run():
        if prologue:
            return run_pro(w, x, direction, c, algo="chunked")
        return run_gpu(w, x, direction, "chunked")

    with G.tuning(segment_tokens=192, no_strip_scan=True):
        with G.tuning(form_inverse=True):
            a = run()
        b = run()
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    args = features(x) if prologue else list(oracle_args(x)[0])
    ro, rH = O.forward(direction, *args, x["h0"], key_scale=c)
    eo, eh = rel_err(b[0], ro), rel_err(b[1], rH)
    print(f"[parity] inverse reuse {direction} prologue={prologue}: out {eo:.3e} state {eh:.3e}", flush=True)
    assert eo <= TOL["bf16"] and eh <= TOL["bf16"], (eo, eh)


# ---------------------------------------------------------------- every head width

DIMS = [16, 32, 48, 80, 96]


@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("direction", ["fwd", "bwd", "bidir"])
def test_chunked_every_head_width(d, direction):
    """The chunked path's other instantiations (d = 64 and 112 run above):
    300 tokens in segments of 128 (three segments, the last ragged), so the
    maps, the chain and the outputs of every width are exercised."""
    w = WORKLOADS[4].resized(frames=2, tokens_per_frame=150, heads=3, d_k=d, d_v=d)
    x = make_inputs(w, 40 + d)
    with G.tuning(segment_tokens=128, no_strip_scan=True):
        check(w, x, direction, "chunked")


# ---------------------------------------------------------------- strip scan

def run_both(w, x, direction, out_dtype=None):
    """The strip scan (the default for short single-scan calls) and segment
    maps with their chain, on the same inputs."""
    a = run_gpu(w, x, direction, "chunked", out_dtype)
    with G.tuning(no_strip_scan=True):
        b = run_gpu(w, x, direction, "chunked", out_dtype)
    return a, b


@pytest.mark.parametrize("d", DIMS + [64, 112])
@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_strip_scan_every_head_width(d, direction):
    """Short forward- and backward-only calls take the strip scan: 300 tokens
    (4 whole sub-chunks and a ragged one), batch 2, per-frame gates and an
    initial state, every head width; against the oracle, and close to the
    segment path (the same rounding points, sums in another order)."""
    w = WORKLOADS[4].resized(batch=2, frames=2, tokens_per_frame=150, heads=3, d_k=d, d_v=d)
    x = make_inputs(w, 140 + d)
    (o, hT), (so, sH) = run_both(w, x, direction)
    ro, rH = O.forward(direction, *oracle_args(x)[0], x["h0"])
    eo, eh = rel_err(o, ro), rel_err(hT, rH)
    print(f"[parity] strip scan d={d} {direction}: out {eo:.3e} state {eh:.3e}", flush=True)
    assert eo <= TOL["bf16"] and eh <= TOL["bf16"], (eo, eh)
    assert rel_err(o, so) <= 1e-2 and rel_err(hT, sH) <= 1e-2


@pytest.mark.parametrize("T", [1, 63, 64, 65, 880, 2048])
def test_strip_scan_lengths(T):
    """One frame of T tokens at d = 112 (the streaming shape, 2 heads):
    from a single token to the longest call that takes the strip scan (32
    sub-chunks)."""
    w = WORKLOADS[3].resized(frames=1, tokens_per_frame=T, heads=2, h0_sigma=0.1)
    x = make_inputs(w, 150 + T)
    for direction in ("fwd", "bwd"):
        check(w, x, direction, "chunked")


def test_strip_scan_bf16_output_and_degenerate_gates():
    """bf16 outputs (the fp32 result rounded once: the bar widens by
    2^-8 max|ref| / RMS(ref)) and the degenerate gates through the strip scan."""
    w = WORKLOADS[3].resized(frames=1, tokens_per_frame=700, heads=2, h0_sigma=0.1)
    x = make_inputs(w, 160)
    o, hT = run_gpu(w, x, "fwd", "chunked", out_dtype=torch.bfloat16)
    ro, rH = O.fwd(*oracle_args(x)[0], x["h0"])
    bound = TOL["bf16"] + 2.0 ** -8 * np.max(np.abs(ro)) / np.sqrt(np.mean(ro * ro))
    assert rel_err(o, ro) <= bound and rel_err(hT, rH) <= TOL["bf16"]
    for case in ("beta0", "nodecay", "strongdecay", "beta1"):
        y = {k: v.copy() for k, v in x.items()}
        if case == "beta0":
            y["beta"][:] = 0.0
        elif case == "nodecay":
            y["log_gate"][:] = 0.0
        elif case == "strongdecay":
            y["log_gate"][:] = -20.0
        else:
            y["beta"][:] = 1.0
        o, hT = run_gpu(w, y, "fwd", "chunked")
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(hT))
        ro, rH = O.fwd(*oracle_args(y)[0], y["h0"])
        eo, eh = rel_err(o, ro), rel_err(hT, rH)
        print(f"[parity] strip scan degenerate {case}: out {eo:.3e} state {eh:.3e}", flush=True)
        assert eo <= TOL["bf16"] and eh <= TOL["bf16"], (case, eo, eh)


@pytest.mark.parametrize("d", DIMS)
def test_jacobi_every_head_width(d):
    w = WORKLOADS[4].resized(frames=3, tokens_per_frame=70, heads=2, d_k=d, d_v=d)
    x = make_inputs(w, 50 + d)
    o, hT = run_jacobi(w, x, "bidir")
    ro, rH = O.jacobi_bidir(*oracle_args(x)[0], x["h0"], key_scale=w.tokens_per_frame ** -0.5,
                            tokens_per_frame=w.tokens_per_frame)
    assert rel_err(o, ro) <= TOL["bf16"] and rel_err(hT, rH) <= TOL["bf16"]


@pytest.mark.parametrize("dk,dv", [(32, 64), (64, 16), (128, 128), (112, 48)])
def test_recurrent_unequal_and_widest_head(dk, dv):
    """The token-recurrent path takes d_k != d_v and d = 128 (fp32, bar 1e-4)."""
    w = WORKLOADS[0].resized(frames=2, tokens_per_frame=24, heads=2, d_k=dk, d_v=dv, h0_sigma=0.1)
    x = make_inputs(w, 60)
    for direction in ("fwd", "bidir"):
        check(w, x, direction, "auto")


@pytest.mark.parametrize("d", [16, 48, 128])
def test_feature_prologue_other_widths_recurrent(d):
    w = WORKLOADS[0].resized(frames=2, tokens_per_frame=24, heads=2, d_k=d, d_v=d, qk_spread=1.0)
    x = make_inputs(w, 70)
    o, hT = run_pro(w, x, "bidir", d ** -0.5)
    ro, rH = O.forward("bidir", *features(x), x["h0"], key_scale=d ** -0.5)
    assert rel_err(o, ro) <= TOL["f32"] and rel_err(hT, rH) <= TOL["f32"]


def test_many_segments_and_heads():
    """Many (batch, head) pairs and segments of 64 tokens (the shortest):
    B = 3, H = 7, 4 frames of 97 tokens (388 tokens, 7 segments)."""
    w = WORKLOADS[4].resized(batch=3, heads=7, frames=4, tokens_per_frame=97)
    x = make_inputs(w, 80)
    with G.tuning(segment_tokens=64, no_strip_scan=True):
        for direction in ("fwd", "bidir"):
            check(w, x, direction, "chunked")


# ---------------------------------------------------------------- degenerate sizes

@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("direction", ["fwd", "bwd", "bidir"])
def test_single_token_sequence(algo, direction):
    """T = 1: one frame of one token (the shortest sequence)."""
    w = WORKLOADS[4].resized(frames=1, tokens_per_frame=1, heads=3)
    check(w, make_inputs(w, 100), direction, algo)


@pytest.mark.parametrize("direction", ["fwd", "bidir"])
def test_jacobi_many_one_token_frames(direction):
    """200 frames of one token: the frame-level chain is 200 maps long (split
    automatically), and a frame of one token equals the token-wise step."""
    w = WORKLOADS[4].resized(frames=200, tokens_per_frame=1, heads=2)
    x = make_inputs(w, 101)
    o, hT = run_jacobi(w, x, direction)
    ro, rH = O.jacobi_forward(direction, *oracle_args(x)[0], x["h0"], key_scale=1.0,
                              tokens_per_frame=1)
    assert rel_err(o, ro) <= TOL["bf16"] and rel_err(hT, rH) <= TOL["bf16"]


@pytest.mark.parametrize("case", ["beta0", "nodecay", "strongdecay", "beta1"])
@pytest.mark.parametrize("algo", ALGOS)
def test_degenerate_gates(case, algo):
    """The method's degenerate gates: beta = 0 (no writes: the initial state,
    decayed, is only read), g = 0 (no decay), g = -20 (the state forgets at
    once: every exp(G) underflows to 0 inside a 64-token block) and beta = 1."""
    w = WORKLOADS[4].resized(frames=3, tokens_per_frame=100, heads=2)
    x = make_inputs(w, 110)
    if case == "beta0":
        x["beta"][:] = 0.0
    elif case == "nodecay":
        x["log_gate"][:] = 0.0
    elif case == "strongdecay":
        x["log_gate"][:] = -20.0
    else:
        x["beta"][:] = 1.0
    o, hT = run_gpu(w, x, "bidir", algo)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(hT))
    ro, rH = O.bidir(*oracle_args(x)[0], x["h0"])
    eo, eh = rel_err(o, ro), rel_err(hT, rH)
    print(f"[parity] degenerate {case} {algo}: out {eo:.3e} state {eh:.3e}", flush=True)
    assert eo <= TOL["bf16"] and eh <= TOL["bf16"], (eo, eh)


# ---------------------------------------------------------------- split chain

@pytest.mark.parametrize("group", [2, 3, 7])
@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_split_chain_chunked(group, direction):
    """The chain of segment maps split into groups (composed in parallel,
    chained, expanded) agrees with the oracle and with the whole chain:
    600 tokens in segments of 64 (10 segments, 9 chain steps)."""
    w = WORKLOADS[4].resized(frames=4, tokens_per_frame=150, heads=3)
    x = make_inputs(w, 90 + group)
    with G.tuning(segment_tokens=64, chain_group=1, no_strip_scan=True):
        whole = run_gpu(w, x, direction, "chunked")
    with G.tuning(segment_tokens=64, chain_group=group, no_strip_scan=True):
        split = check(w, x, direction, "chunked")
        o, hT = run_gpu(w, x, direction, "chunked")
    # both are within the bar of the oracle; between them only the chain's
    # rounding differs (start states feed the output kernel's fp16 operands,
    # so a flipped fp16 rounding of a state element shows at ~2^-11 relative)
    assert rel_err(o, whole[0]) <= 1e-2 and rel_err(hT, whole[1]) <= 1e-2, split


@pytest.mark.parametrize("group", [2, 4])
def test_split_chain_jacobi(group):
    w = WORKLOADS[4].resized(frames=11, tokens_per_frame=40, heads=2)
    x = make_inputs(w, 95)
    with G.tuning(chain_group=group):
        o, hT = run_jacobi(w, x, "bidir")
    ro, rH = O.jacobi_bidir(*oracle_args(x)[0], x["h0"], key_scale=w.tokens_per_frame ** -0.5,
                            tokens_per_frame=w.tokens_per_frame)
    assert rel_err(o, ro) <= TOL["bf16"] and rel_err(hT, rH) <= TOL["bf16"]


def test_split_chain_chunk_causal():
    w = WORKLOADS[4].resized(frames=6, tokens_per_frame=100, heads=2)
    x = make_inputs(w, 96)
    with G.tuning(segment_tokens=64, chain_group=3):
        o, hT = run_cc(w, x, 2, 2, "chunked")
    ro, rH = O.chunk_causal(*oracle_args(x)[0], x["h0"], tokens_per_frame=w.tokens_per_frame,
                            first_chunk_frames=2, chunk_frames=2)
    assert rel_err(o, ro) <= TOL["bf16"] and rel_err(hT, rH) <= TOL["bf16"]


# ---------------------------------------------------------------- chunk-causal layer

CC = {
    # name: (workload, first chunk frames, later chunk frames)
    "clip60s_4_3": (WORKLOADS[2].resized(frames=8, heads=2), 4, 3),          # chunks 4, 3, 1
    "ragged_2_2": (WORKLOADS[1].resized(frames=5, tokens_per_frame=201, heads=2), 2, 2),
    "batched_1_1": (WORKLOADS[4].resized(frames=3, heads=3), 1, 1),         # d = 64, initial state
    "one_chunk": (WORKLOADS[1].resized(frames=3, heads=2), 5, 5),           # = bidirectional
}


def run_cc(w, x, first, every, algo, out_dtype=None, qkv=None):
    d = to_device(x, qkv or w.qkv_dtype)
    h0 = d["h0"] if np.any(x["h0"]) else None
    out, hT = G.forward(d["q"], d["k"], d["v"], d["log_gate"], d["beta"], h0, "chunk_causal",
                        tokens_per_frame=w.tokens_per_frame, algo=algo, out_dtype=out_dtype,
                        first_chunk_frames=first, chunk_frames=every)
    torch.cuda.synchronize()
    return to_numpy(out), to_numpy(hT)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("name", list(CC))
def test_chunk_causal_bf16(algo, name):
    w, first, every = CC[name]
    x = make_inputs(w, 11)
    o, hT = run_cc(w, x, first, every, algo)
    ro, rH = O.chunk_causal(*oracle_args(x)[0], x["h0"], tokens_per_frame=w.tokens_per_frame,
                            first_chunk_frames=first, chunk_frames=every)
    eo, eh = rel_err(o, ro), rel_err(hT, rH)
    print(f"[parity] {w.name} chunk-causal {first},{every} {algo}: out {eo:.3e} state {eh:.3e}", flush=True)
    assert eo <= TOL["bf16"] and eh <= TOL["bf16"], (eo, eh)


def test_chunk_causal_fp32_recurrent():
    w = WORKLOADS[0]
    x = make_inputs(w, 12)
    o, hT = run_cc(w, x, 2, 1, "auto")
    ro, rH = O.chunk_causal(*oracle_args(x)[0], x["h0"], tokens_per_frame=w.tokens_per_frame,
                            first_chunk_frames=2, chunk_frames=1)
    assert rel_err(o, ro) <= TOL["f32"] and rel_err(hT, rH) <= TOL["f32"]


def test_chunk_causal_bf16_output_and_schedules():
    """bf16 output through the fp32 partial; the concurrent and in-order
    schedules give bit-identical results."""
    w, first, every = CC["clip60s_4_3"]
    x = make_inputs(w, 13)
    with G.tuning(segment_tokens=512):
        a = run_cc(w, x, first, every, "chunked", out_dtype=torch.bfloat16)
        with G.tuning(serial_scans=True):
            b = run_cc(w, x, first, every, "chunked", out_dtype=torch.bfloat16)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    ro, rH = O.chunk_causal(*oracle_args(x)[0], x["h0"], tokens_per_frame=w.tokens_per_frame,
                            first_chunk_frames=first, chunk_frames=every)
    bound = TOL["bf16"] + 2.0 ** -8 * np.max(np.abs(ro)) / np.sqrt(np.mean(ro * ro))
    assert rel_err(a[0], ro) <= bound and rel_err(a[1], rH) <= TOL["bf16"]


# ---------------------------------------------------------------- frame-level (Jacobi) transition

JAC = {
    "clip60s": WORKLOADS[2].resized(frames=3, heads=3),
    "ragged": WORKLOADS[1].resized(frames=4, tokens_per_frame=201, heads=2),
    "batched": WORKLOADS[4].resized(frames=3, heads=3),     # d = 64, initial state
    "short": WORKLOADS[4].resized(frames=2, tokens_per_frame=5, heads=2, h0_sigma=0.3),
}


def run_jacobi(w, x, direction, out_dtype=None):
    d = to_device(x, w.qkv_dtype)
    h0 = d["h0"] if np.any(x["h0"]) else None
    out, hT = G.forward(d["q"], d["k"], d["v"], d["log_gate"], d["beta"], h0, direction,
                        tokens_per_frame=w.tokens_per_frame, key_scale=w.tokens_per_frame ** -0.5,
                        intra="jacobi", out_dtype=out_dtype)
    torch.cuda.synchronize()
    return to_numpy(out), to_numpy(hT)


@pytest.mark.parametrize("name", list(JAC))
@pytest.mark.parametrize("direction", ["fwd", "bwd", "bidir"])
def test_jacobi_bf16(name, direction):
    """The frame-level transition against the oracle's (key scale 1/sqrt(S),
    the pages' spatial scale for unit-norm keys)."""
    w = JAC[name]
    x = make_inputs(w, 7)
    o, hT = run_jacobi(w, x, direction)
    a, h0 = oracle_args(x)
    ro, rH = O.jacobi_forward(direction, *a, h0, key_scale=w.tokens_per_frame ** -0.5,
                              tokens_per_frame=w.tokens_per_frame)
    eo, eh = rel_err(o, ro), rel_err(hT, rH)
    print(f"[parity] {w.name} jacobi {direction}: out {eo:.3e} state {eh:.3e}", flush=True)
    assert eo <= TOL["bf16"] and eh <= TOL["bf16"], (eo, eh)


def test_jacobi_step_chain_matches_forward():
    """gdn_step with the frame-level transition, frame after frame with the
    state carried in place, equals the whole-sequence forward scan."""
    w = JAC["clip60s"].resized(h0_sigma=0.1)
    x = make_inputs(w, 8)
    d = to_device(x, w.qkv_dtype)
    S, c = w.tokens_per_frame, w.tokens_per_frame ** -0.5
    state = d["h0"].clone()
    outs = []
    for f in range(w.frames):
        sl = slice(f * S, (f + 1) * S)
        o, _ = G.step(*(d[n][:, sl].contiguous() for n in ("q", "k", "v", "log_gate", "beta")),
                      state, state, key_scale=c, intra="jacobi")
        outs.append(o)
    o = to_numpy(torch.cat(outs, dim=1))
    ro, rH = O.jacobi(*oracle_args(x)[0], x["h0"], key_scale=c, tokens_per_frame=S)
    assert rel_err(o, ro) <= TOL["bf16"] and rel_err(to_numpy(state), rH) <= TOL["bf16"]
    fo, fH = run_jacobi(w, x, "fwd")
    assert np.array_equal(o, fo) and np.array_equal(to_numpy(state), fH)


def test_jacobi_bf16_output():
    w = JAC["batched"]
    x = make_inputs(w, 9)
    o, hT = run_jacobi(w, x, "bidir", out_dtype=torch.bfloat16)
    ro, rH = O.jacobi_bidir(*oracle_args(x)[0], x["h0"], key_scale=w.tokens_per_frame ** -0.5,
                            tokens_per_frame=w.tokens_per_frame)
    bound = TOL["bf16"] + 2.0 ** -8 * np.max(np.abs(ro)) / np.sqrt(np.mean(ro * ro))
    assert rel_err(o, ro) <= bound and rel_err(hT, rH) <= TOL["bf16"]


# ---------------------------------------------------------------- feature prologue

PRO = {
    # name: (workload with raw q/k, key scale)
    "clip60s": (WORKLOADS[2].resized(frames=3, heads=3, qk_spread=1.0), (112 * 880) ** -0.5),
    "ragged": (WORKLOADS[1].resized(frames=3, tokens_per_frame=201, heads=2, qk_spread=1.0), 112 ** -0.5),
    "batched": (WORKLOADS[4].resized(frames=2, heads=3, qk_spread=1.0), (64 * 880) ** -0.5),
}


def features(x):
    """Oracle inputs with the prologue applied on the CPU (float64)."""
    a = [x[n] for n in ("q", "k", "v", "log_gate", "beta")]
    a[0], a[1] = O.query_features(a[0]), O.key_features(a[1])
    return a


def run_pro(w, x, direction, c, algo="auto", intra="sequential", out_dtype=None, chunks=(0, 0)):
    d = to_device(x, w.qkv_dtype)
    h0 = d["h0"] if np.any(x["h0"]) else None
    out, hT = G.forward(d["q"], d["k"], d["v"], d["log_gate"], d["beta"], h0, direction,
                        tokens_per_frame=w.tokens_per_frame, key_scale=c, algo=algo, intra=intra,
                        out_dtype=out_dtype, prologue="features", first_chunk_frames=chunks[0],
                        chunk_frames=chunks[1])
    torch.cuda.synchronize()
    return to_numpy(out), to_numpy(hT)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("name", list(PRO))
@pytest.mark.parametrize("direction", ["fwd", "bwd", "bidir"])
def test_feature_prologue_bf16(algo, name, direction):
    """Raw q/k through the fused prologue against the oracle applied to
    key_features(k), query_features(q)."""
    w, c = PRO[name]
    x = make_inputs(w, 31)
    o, hT = run_pro(w, x, direction, c, algo=algo)
    ro, rH = O.forward(direction, *features(x), x["h0"], key_scale=c)
    eo, eh = rel_err(o, ro), rel_err(hT, rH)
    print(f"[parity] {w.name} prologue {direction} {algo}: out {eo:.3e} state {eh:.3e}", flush=True)
    assert eo <= TOL["bf16"] and eh <= TOL["bf16"], (eo, eh)


def test_feature_prologue_fp32_recurrent():
    w = WORKLOADS[0].resized(qk_spread=1.0)
    x = make_inputs(w, 32)
    for direction in ("fwd", "bidir"):
        o, hT = run_pro(w, x, direction, 16 ** -0.5)
        ro, rH = O.forward(direction, *features(x), x["h0"], key_scale=16 ** -0.5)
        assert rel_err(o, ro) <= TOL["f32"] and rel_err(hT, rH) <= TOL["f32"]


@pytest.mark.parametrize("direction", ["fwd", "bidir"])
def test_feature_prologue_jacobi(direction):
    w, c = PRO["clip60s"]
    x = make_inputs(w, 33)
    o, hT = run_pro(w, x, direction, c, intra="jacobi")
    ro, rH = O.jacobi_forward(direction, *features(x), x["h0"], key_scale=c, tokens_per_frame=w.tokens_per_frame)
    eo, eh = rel_err(o, ro), rel_err(hT, rH)
    print(f"[parity] {w.name} prologue jacobi {direction}: out {eo:.3e} state {eh:.3e}", flush=True)
    assert eo <= TOL["bf16"] and eh <= TOL["bf16"], (eo, eh)


@pytest.mark.parametrize("algo", ALGOS)
def test_feature_prologue_chunk_causal(algo):
    w, c = PRO["ragged"]
    x = make_inputs(w, 34)
    o, hT = run_pro(w, x, "chunk_causal", c, algo=algo, chunks=(2, 1))
    ro, rH = O.chunk_causal(*features(x), x["h0"], key_scale=c, tokens_per_frame=w.tokens_per_frame,
                            first_chunk_frames=2, chunk_frames=1)
    assert rel_err(o, ro) <= TOL["bf16"] and rel_err(hT, rH) <= TOL["bf16"]


@pytest.mark.parametrize("algo", ALGOS)
def test_feature_prologue_step_chain_matches_forward(algo):
    """gdn_step with the prologue, frame after frame, against the forward scan:
    the factors are per token, so framing cannot change them; the token-recurrent
    path then agrees bit for bit, the chunked one (whose 64-token blocks start
    at each call's first token) to rounding."""
    w, c = PRO["batched"]
    x = make_inputs(w, 35)
    d = to_device(x, w.qkv_dtype)
    S = w.tokens_per_frame
    state = d["h0"].clone()
    outs = []
    for f in range(w.frames):
        sl = slice(f * S, (f + 1) * S)
        o, _ = G.step(*(d[n][:, sl].contiguous() for n in ("q", "k", "v", "log_gate", "beta")),
                      state, state, key_scale=c, prologue="features", algo=algo)
        outs.append(o)
    o = to_numpy(torch.cat(outs, dim=1))
    fo, fH = run_pro(w, x, "fwd", c, algo=algo)
    if algo == "recurrent":
        assert np.array_equal(o, fo) and np.array_equal(to_numpy(state), fH)
    else:
        assert rel_err(o, fo) <= 1e-2 and rel_err(to_numpy(state), fH) <= 1e-2
    ro, rH = O.fwd(*features(x), x["h0"], key_scale=c)
    assert rel_err(o, ro) <= TOL["bf16"] and rel_err(fH, rH) <= TOL["bf16"]


def test_feature_prologue_is_invariant_to_token_magnitudes():
    """Property at any size: the features do not depend on a positive factor
    per (token, head) of the raw q and k (powers of two keep bf16 exact); the
    results agree to rounding and to the epsilon, which is not scaled (hence
    factors >= 1 only)."""
    w, c = PRO["clip60s"]
    x = make_inputs(w, 36)
    rng = np.random.default_rng(37)
    y = dict(x)
    for n in ("q", "k"):
        y[n] = (x[n] * 2.0 ** rng.integers(0, 4, x[n].shape[:3] + (1,))).astype(np.float32)
    a, b = run_pro(w, x, "bidir", c), run_pro(w, y, "bidir", c)
    assert rel_err(a[0], b[0]) <= 5e-3 and rel_err(a[1], b[1]) <= 5e-3


FULL = [(1, "bidir", [0, 19]), (1, "fwd", [5]), (2, "bidir", [7]), (2, "fwd", [13]),
        (4, "bidir", [(0, 3), (1, 34)]), (4, "fwd", [(1, 20)])]


@pytest.mark.slow
@pytest.mark.parametrize("algo", ["chunked"])
@pytest.mark.parametrize("idx,direction,heads", FULL)
def test_full_size_sampled_heads(algo, idx, direction, heads):
    """Full workload sizes in the bench's launch configuration; the oracle is
    run on sampled (batch, head) pairs over the whole sequence."""
    w = WORKLOADS[idx]
    x = make_inputs(w, 0)
    o, hT = run_gpu(w, x, direction, algo)
    tol = TOL[w.qkv_dtype]
    for hh in heads:
        b, h = (hh if isinstance(hh, tuple) else (0, hh))
        a = [t[b:b + 1, :, h:h + 1] for t in (x["q"], x["k"], x["v"], x["log_gate"], x["beta"])]
        ro, rH = O.forward(direction, *a, x["h0"][b:b + 1, h:h + 1])
        eo = rel_err(o[b:b + 1, :, h:h + 1], ro)
        eh = rel_err(hT[b:b + 1, h:h + 1], rH)
        print(f"[parity-full] {w.name} {direction} b{b} h{h}: out {eo:.3e} state {eh:.3e}",
              flush=True)
        assert eo <= tol and eh <= tol


@pytest.mark.slow
def test_full_size_feature_prologue_sampled_head():
    """The 60 s clip with raw q/k through the prologue (bidirectional, key
    scale 1/sqrt(D*S)) in the bench's launch configuration; head 5 against
    the oracle over the whole sequence."""
    w = WORKLOADS[2].resized(qk_spread=1.0)
    c = (w.d_k * w.tokens_per_frame) ** -0.5
    x = make_inputs(w, 0)
    o, hT = run_pro(w, x, "bidir", c, algo="chunked")
    h = 5
    a = [t[:, :, h:h + 1] for t in features(x)]
    ro, rH = O.bidir(*a, x["h0"][:, h:h + 1], key_scale=c)
    eo, eh = rel_err(o[:, :, h:h + 1], ro), rel_err(hT[:, h:h + 1], rH)
    print(f"[parity-full] {w.name} prologue bidir h{h}: out {eo:.3e} state {eh:.3e}", flush=True)
    assert eo <= TOL["bf16"] and eh <= TOL["bf16"]


@pytest.mark.slow
def test_full_size_stream_121_steps_sampled_heads():
    """The chunk-causal streaming workload at full size: 121 gdn_step calls of
    one 880-token frame each on 20 heads x 112 with the long-memory gates, the
    fp32 state carried in place between calls, in the launch configuration the
    bench times.  Two sampled heads' outputs (all 106,480 tokens) and final
    states against the oracle's forward scan over the whole sequence."""
    w = WORKLOADS[3]
    x = make_inputs(w, 0)
    d = to_device(x, w.qkv_dtype)
    S = w.tokens_per_frame
    state = torch.zeros((w.batch, w.heads, w.d_k, w.d_v), dtype=torch.float32, device="cuda")
    out = torch.empty((w.batch, w.tokens, w.heads, w.d_v), dtype=torch.float32, device="cuda")
    for f in range(w.frames):
        sl = slice(f * S, (f + 1) * S)
        G.step(*(d[n][:, sl] for n in ("q", "k", "v", "log_gate", "beta")), state, state, out=out[:, sl])
    torch.cuda.synchronize()
    o, hT = to_numpy(out), to_numpy(state)
    for h in (4, 17):
        a = [t[:, :, h:h + 1] for t in (x["q"], x["k"], x["v"], x["log_gate"], x["beta"])]
        ro, rH = O.fwd(*a, x["h0"][:, h:h + 1])
        eo, eh = rel_err(o[:, :, h:h + 1], ro), rel_err(hT[:, h:h + 1], rH)
        print(f"[parity-full] {w.name} 121 steps h{h}: out {eo:.3e} state {eh:.3e}", flush=True)
        assert eo <= TOL["bf16"] and eh <= TOL["bf16"], (h, eo, eh)


def test_chunked_at_the_edge_of_its_fp16_domain():
    """The chunked path's documented range: values scaled by 2^11 (exact in
    bf16) so that outputs reach about 1e4 and the fp16 partial of the
    bidirectional sum about that too; the relative error is that of the
    unscaled inputs (the layer is linear in v and the initial state)."""
    w = SMALL["batched"]
    x = make_inputs(w, 120)
    x["v"] = x["v"] * 2.0 ** 11
    x["h0"] = x["h0"] * 2.0 ** 11
    with G.tuning(segment_tokens=192):
        o, hT = run_gpu(w, x, "bidir", "chunked")
    ro, rH = O.bidir(*oracle_args(x)[0], x["h0"])
    assert 4e3 < np.max(np.abs(ro)) < 3e4, np.max(np.abs(ro))
    eo, eh = rel_err(o, ro), rel_err(hT, rH)
    print(f"[parity] fp16 domain edge: max|out| {np.max(np.abs(ro)):.3g}, out {eo:.3e} state {eh:.3e}", flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(hT))
    assert eo <= TOL["bf16"] and eh <= TOL["bf16"], (eo, eh)


@pytest.mark.parametrize("direction", ["fwd", "bidir"])
def test_recurrent_takes_bf16_values_beyond_fp16(direction):
    """Values past fp16's range (v scaled by 2^17, so |v| reaches about 5e5):
    the token-recurrent path computes in fp32 throughout and stays within the
    bf16 bar."""
    w = SMALL["clip5s"]
    x = make_inputs(w, 121)
    x["v"] = x["v"] * 2.0 ** 17
    assert np.max(np.abs(x["v"])) > 65504
    o, hT = run_gpu(w, x, direction, "recurrent")
    ro, rH = O.forward(direction, *oracle_args(x)[0], x["h0"])
    eo, eh = rel_err(o, ro), rel_err(hT, rH)
    print(f"[parity] beyond fp16 {direction}: max|v| {np.max(np.abs(x['v'])):.3g}, out {eo:.3e} state {eh:.3e}",
          flush=True)
    assert eo <= TOL["bf16"] and eh <= TOL["bf16"], (eo, eh)


def test_binding_checks_out_and_workspace():
    """A supplied ``out`` sets the output dtype (bf16 here: the fp32 result
    rounded once); a wrong shape, a dtype that contradicts ``out_dtype``, or a
    workspace on another device raise before anything is enqueued."""
    w = SMALL["clip60s"]
    x = make_inputs(w, 122)
    d = to_device(x, w.qkv_dtype)
    args = [d[n] for n in ("q", "k", "v", "log_gate", "beta")]
    kw = dict(tokens_per_frame=w.tokens_per_frame)
    ref, _ = G.forward(*args, None, "bidir", **kw)
    out = torch.empty(ref.shape, dtype=torch.bfloat16, device="cuda")
    o, _ = G.forward(*args, None, "bidir", out=out, **kw)
    torch.cuda.synchronize()
    assert o is out and o.dtype == torch.bfloat16
    assert torch.equal(o, ref.to(torch.bfloat16))
    with pytest.raises(ValueError):
        G.forward(*args, None, "bidir", out=torch.empty(ref.shape[:-1] + (8,), device="cuda"), **kw)
    with pytest.raises(TypeError):
        G.forward(*args, None, "bidir", out=out, out_dtype=torch.float32, **kw)
    with pytest.raises(ValueError):
        G.forward(*args, None, "bidir", workspace=torch.empty(1 << 20, dtype=torch.uint8), **kw)
    with pytest.raises(ValueError):
        G.forward(*args, None, "bidir", out=torch.empty(ref.shape, device="cuda").transpose(1, 2).contiguous()
                  .transpose(1, 2), **kw)
