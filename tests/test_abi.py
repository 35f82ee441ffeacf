"""libgdn's C ABI on the host: exports, version, status text, workspace sizing
and argument validation.  No compute call is made, so no GPU is needed: every
check below fails (or sizes) before the library makes any HIP call."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_frame_amd as G

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = G.lib()
    names = declared_functions()
    assert {"gdn_forward", "gdn_step", "gdn_workspace_size"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"{n} declared in gdn.h but not exported"


def test_version_and_status_strings():
    L = G.lib()
    assert L.gdn_abi_version() == G.ABI_VERSION == 2
    for s, text in enumerate(["GDN_OK", "GDN_ERR_INVALID_ARGUMENT", "GDN_ERR_UNSUPPORTED",
                              "GDN_ERR_WORKSPACE_TOO_SMALL", "GDN_ERR_HIP"]):
        assert L.gdn_status_string(s).decode() == text
    assert L.gdn_status_string(99).decode() == "GDN_ERR_UNKNOWN_STATUS"


def prob(**kw):
    base = dict(batch=1, heads=2, d_k=64, d_v=64, frames=3, tokens_per_frame=100,
                qkv_dtype=G.BF16, out_dtype=G.BF16, algo="auto")
    base.update(kw)
    return G.make_problem(**base)


def test_recurrent_workspace_is_the_bidirectional_accumulator():
    p = prob(algo="recurrent")
    assert G.workspace_size(p, "fwd") == 0
    assert G.workspace_size(p, "bwd") == 0
    assert G.workspace_size(p, "bidir") == 1 * 300 * 2 * 64 * 4


@pytest.mark.parametrize("field,value", [
    ("abi_version", 1), ("abi_version", 3), ("batch", 0), ("heads", -1), ("frames", 0), ("tokens_per_frame", 0),
    ("d_k", 20), ("d_k", 144), ("d_v", 8), ("qkv_dtype", 7), ("out_dtype", -1), ("algo", 9),
    ("segment_tokens", -64), ("chain_group", -1), ("flags", 8), ("flags", -1),
])
def test_bad_problem_fields_are_rejected(field, value):
    p = prob()
    setattr(p, field, value)
    with pytest.raises(G.GdnError) as e:
        G.workspace_size(p, "bidir")
    assert e.value.status == G.ERR_INVALID_ARGUMENT
    assert G.lib().gdn_last_error_message().decode() != ""


def test_reserved_and_key_scale_and_direction_checks():
    for i in range(5):
        p = prob()
        p.reserved[i] = 1
        with pytest.raises(G.GdnError):
            G.workspace_size(p, "bidir")
    p = prob(key_scale=float("nan"))
    with pytest.raises(G.GdnError):
        G.workspace_size(p, "bidir")
    n = ctypes.c_size_t()
    assert G.lib().gdn_workspace_size(ctypes.byref(prob()), 7, ctypes.byref(n)) == G.ERR_INVALID_ARGUMENT
    assert G.lib().gdn_workspace_size(None, 0, ctypes.byref(n)) == G.ERR_INVALID_ARGUMENT
    assert G.lib().gdn_workspace_size(ctypes.byref(prob()), 0, None) == G.ERR_INVALID_ARGUMENT


FAKE = 0x10000  # never dereferenced: validation fails before any use


def call_forward(p, direction=G.BIDIRECTIONAL, q=FAKE, k=FAKE, v=FAKE, g=FAKE, b=FAKE, h0=None,
                 out=FAKE, hT=None, ws=None, ws_bytes=0):
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return G.lib().gdn_forward(ctypes.byref(p), direction, vp(q), vp(k), vp(v), vp(g), vp(b),
                               vp(h0), vp(out), vp(hT), vp(ws), ws_bytes, None)


def test_forward_rejects_null_and_misaligned_pointers_without_launching():
    p = prob(algo="recurrent")
    for name in ("q", "k", "v", "g", "b", "out"):
        assert call_forward(p, **{name: None}) == G.ERR_INVALID_ARGUMENT
        assert call_forward(p, **{name: FAKE + 2}) == G.ERR_INVALID_ARGUMENT
    assert call_forward(p, h0=FAKE + 4) == G.ERR_INVALID_ARGUMENT
    assert call_forward(p, direction=5) == G.ERR_INVALID_ARGUMENT


def test_forward_rejects_small_workspace():
    p = prob(algo="recurrent")
    assert call_forward(p) == G.ERR_WORKSPACE_TOO_SMALL
    need = G.workspace_size(p, "bidir")
    assert call_forward(p, ws=FAKE, ws_bytes=need - 1) == G.ERR_WORKSPACE_TOO_SMALL
    assert "needed" in G.lib().gdn_last_error_message().decode()


def test_step_requires_one_frame_and_state_out():
    L = G.lib()
    vp = ctypes.c_void_p
    p = prob(frames=2, algo="recurrent")
    args = [vp(FAKE)] * 5
    assert L.gdn_step(ctypes.byref(p), *args, None, vp(FAKE), vp(FAKE), None, 0, None) \
        == G.ERR_INVALID_ARGUMENT
    p = prob(frames=1, algo="recurrent")
    assert L.gdn_step(ctypes.byref(p), *args, None, None, vp(FAKE), None, 0, None) \
        == G.ERR_INVALID_ARGUMENT
    assert "state_out" in L.gdn_last_error_message().decode()


def test_frame_level_transition_validation_and_workspace():
    """intra must be SEQUENTIAL or JACOBI; JACOBI needs bf16 q/k/v, d_k = d_v
    <= 112 and no token-recurrent algorithm; its workspace holds maps and
    states for every frame boundary of each scan."""
    p = prob()
    p.intra = 2
    with pytest.raises(G.GdnError) as e:
        G.workspace_size(p, "bidir")
    assert e.value.status == G.ERR_INVALID_ARGUMENT
    for kw in (dict(qkv_dtype=G.F32), dict(d_v=32), dict(d_k=128, d_v=128), dict(algo="recurrent")):
        p = prob(intra="jacobi", **kw)
        with pytest.raises(G.GdnError) as e:
            G.workspace_size(p, "fwd")
        assert e.value.status == G.ERR_UNSUPPORTED, kw
    p = prob(intra="jacobi")      # B = 1, H = 2, d = 64, F = 3
    maps = 2 * 1 * 2 * 4 * 64 * 128 * 4
    states = 2 * 1 * 2 * 4 * 64 * 64 * 4
    assert G.workspace_size(p, "bidir") == maps + states
    assert G.workspace_size(p, "fwd") == (maps + states) // 2
    assert call_forward(p, ws=FAKE, ws_bytes=maps + states - 1) == G.ERR_WORKSPACE_TOO_SMALL


def test_chunk_causal_validation_and_workspace():
    """GDN_CHUNK_CAUSAL needs chunk sizes >= 1 and the token-wise transition;
    its chunked-path workspace holds one scan's maps and states and the fp16
    partial of the reversed chunks, its recurrent one the fp32 partial."""
    n = ctypes.c_size_t()
    p = prob()
    assert G.lib().gdn_workspace_size(ctypes.byref(p), G.CHUNK_CAUSAL, ctypes.byref(n)) == G.ERR_INVALID_ARGUMENT
    p = prob(first_chunk_frames=2, chunk_frames=0)
    assert G.lib().gdn_workspace_size(ctypes.byref(p), G.CHUNK_CAUSAL, ctypes.byref(n)) == G.ERR_INVALID_ARGUMENT
    p = prob(first_chunk_frames=2, chunk_frames=1, intra="jacobi")
    assert G.lib().gdn_workspace_size(ctypes.byref(p), G.CHUNK_CAUSAL, ctypes.byref(n)) == G.ERR_UNSUPPORTED
    p = prob(first_chunk_frames=2, chunk_frames=1, algo="recurrent")
    assert G.workspace_size(p, "chunk_causal") == 1 * 300 * 2 * 64 * 4
    # chunked: the fp16 partial of the reversed chunks, whatever the output dtype
    p32 = prob(first_chunk_frames=2, chunk_frames=1, algo="chunked", out_dtype=G.F32)
    pbf = prob(first_chunk_frames=2, chunk_frames=1, algo="chunked", out_dtype=G.BF16)
    assert G.workspace_size(pbf, "chunk_causal") == G.workspace_size(p32, "chunk_causal")
    tm = 2 * ((300 + 63) // 64) * 5120   # the forward-only call's sub-chunk inverse blocks (5 segments)
    assert G.workspace_size(p32, "chunk_causal") - (G.workspace_size(p32, "fwd") - tm) >= 1 * 300 * 2 * 64 * 2
    assert G.workspace_size(p32, "chunk_causal") < G.workspace_size(p32, "bidir")


def test_feature_prologue_validation_and_workspace():
    """prologue is NONE or FEATURES; FEATURES adds two fp32 factors per
    (token, head) to the workspace of every path and direction (each region
    rounded up to 256 bytes)."""
    p = prob(prologue=2)
    with pytest.raises(G.GdnError) as e:
        G.workspace_size(p, "bidir")
    assert e.value.status == G.ERR_INVALID_ARGUMENT
    fac = 2 * 1 * 2 * (300 + 2) * 4   # (fk, fq) pairs of tokens -1 .. T per (batch, head)
    rounded = (fac + 255) // 256 * 256
    for kw in (dict(algo="recurrent"), dict(algo="chunked"), dict(intra="jacobi"),
               dict(algo="recurrent", qkv_dtype=G.F32)):
        for d in ("fwd", "bwd", "bidir"):
            # (short single-scan calls without the prologue would take the
            # strip scan, whose workspace is laid out differently)
            with G.tuning(no_strip_scan=True):
                a = G.workspace_size(prob(**kw), d)
            b = G.workspace_size(prob(prologue="features", **kw), d)
            if kw == dict(algo="chunked") and d == "bidir":
                # at d_k <= 64 a bidirectional call without the prologue also
                # holds both scans' sub-chunk inverse blocks (5 KB per 64 tokens)
                a -= 2 * 1 * 2 * ((300 + 63) // 64) * 5120
            assert b - a in (fac, rounded), (kw, d, a, b)
    p = prob(prologue="features", first_chunk_frames=2, chunk_frames=1)
    # without the prologue the chunk-causal call at d_k <= 64 holds the forward scan's inverse blocks
    plain = G.workspace_size(prob(first_chunk_frames=2, chunk_frames=1), "chunk_causal") - 2 * 5 * 5120
    assert G.workspace_size(p, "chunk_causal") - plain in (fac, rounded)


def test_split_chain_workspace():
    """A split chain adds group maps and group start states to the workspace;
    the plan is part of the call's problem (no state in the library)."""
    p = prob(frames=40, tokens_per_frame=100, algo="chunked", tuning=G.Tuning(segment_tokens=64, chain_group=1))
    whole = G.workspace_size(p, "fwd")
    whole_bi = G.workspace_size(p, "bidir")
    p4 = prob(frames=40, tokens_per_frame=100, algo="chunked", tuning=G.Tuning(segment_tokens=64, chain_group=4))
    split = G.workspace_size(p4, "fwd")
    assert G.workspace_size(p, "fwd") == whole          # sizing leaves nothing behind
    steps = (40 * 100 + 63) // 64 - 1
    groups = (steps + 3) // 4
    extra = 1 * 2 * groups * 64 * (128 + 64) * 4
    assert split - whole == pytest.approx(extra, abs=512)
    assert G.workspace_size(p4, "bidir") == whole_bi   # bidirectional chains are never split


def test_tuning_context_fills_the_problem():
    """The binding's tuning() context sets the problem's tuning fields for
    calls inside it and restores them after; explicit Tuning wins."""
    assert prob().segment_tokens == 0 and prob().flags == 0
    with G.tuning(segment_tokens=512, serial_scans=True, form_inverse=True):
        p = prob()
        assert (p.segment_tokens, p.chain_group, p.flags) == (512, 0, 3)
        assert prob(tuning=G.Tuning()).flags == 0
        with G.tuning(chain_group=3):
            assert (prob().segment_tokens, prob().chain_group) == (512, 3)
    assert (prob().segment_tokens, prob().chain_group, prob().flags) == (0, 0, 0)


def test_segment_plan_follows_the_problem():
    p = prob(frames=40, tokens_per_frame=100, algo="chunked")
    auto = G.segment_plan(p, "bidir")
    assert auto % 64 == 0 and auto > 0
    assert G.segment_plan(prob(frames=40, tokens_per_frame=100, algo="chunked",
                               tuning=G.Tuning(segment_tokens=100)), "bidir") == 128
    assert G.segment_plan(prob(algo="recurrent"), "bidir") == 0


def _plan_steps(hb, U, ns):
    """Launch time of a segment count in sub-chunk steps: the busiest of the
    8 XCDs (32 CUs each) holds hb * ceil(ns / 8) workgroups, one per CU, each
    ceil(U / ns) sub-chunks plus one step to start."""
    return -(-hb * -(-ns // 8) // 32) * (-(-U // ns) + 1)


@pytest.mark.parametrize("B,H,d,F,S,want", [
    (1, 20, 112, 121, 880, 1664),   # the 60 s clip: 64 segments, five whole rounds
    (2, 35, 64, 121, 880, 2688),    # the batched workload: 40 segments
    (1, 20, 112, 21, 880, 832),     # the 5 s clip: 23 segments
    (1, 20, 112, 3, 880, 384),      # three frames: 7 segments (the 2 sqrt(U) cap leaves 1..8)
])
def test_automatic_segment_plan(B, H, d, F, S, want):
    """The automatic segment length takes the count with the fewest launch
    steps (_plan_steps) among 1..8 and multiples of 8, at most about 2 sqrt(U)
    for U sub-chunks, the smaller count on ties; forward and bidirectional
    calls plan alike."""
    p = G.make_problem(batch=B, heads=H, d_k=d, d_v=d, frames=F, tokens_per_frame=S, qkv_dtype=G.BF16,
                       algo="chunked", tuning=G.Tuning(no_strip_scan=True))
    T = F * S
    U = -(-T // 64)
    assert G.segment_plan(p, "bidir") == want == G.segment_plan(p, "fwd")
    cap = 1
    while (cap + 1) ** 2 <= 4 * U:
        cap += 1
    cands = [n for n in range(1, cap + 1) if n <= 8 or n % 8 == 0]
    best = min(cands, key=lambda n: (_plan_steps(B * H, U, n), n))
    assert want == -(-(-(-T // best)) // 64) * 64


def test_inverse_reuse_workspace():
    """A forward-only chunked call with more than one segment holds 5 KB of
    fp16 inverse blocks per 64-token sub-chunk and head, whether or not the
    output kernel loads them; a bidirectional call holds them for both scans
    at d_k <= 64 and none at larger widths."""
    def p_(seg, form=False):   # 4000 tokens: 63 sub-chunks
        return prob(frames=40, tokens_per_frame=100, algo="chunked",
                    tuning=G.Tuning(segment_tokens=seg, chain_group=1, form_inverse=form))
    one = G.workspace_size(p_(4096), "fwd")      # one segment: no maps, no inverse blocks
    one_bi = G.workspace_size(p_(4096), "bidir")
    on = G.workspace_size(p_(512), "fwd")        # 8 segments
    on_bi = G.workspace_size(p_(512), "bidir")
    assert G.workspace_size(p_(512, form=True), "fwd") == on
    per_seg = 2 * 64 * (128 + 64) * 4           # one scan's map and start state, 2 heads
    tm = 2 * 63 * 5120
    assert on - one == pytest.approx(7 * per_seg + tm, abs=1024)
    assert on_bi - one_bi == pytest.approx(2 * 7 * per_seg + 2 * tm, abs=1024)
    wide = dict(frames=40, tokens_per_frame=100, algo="chunked", d_k=96, d_v=96)
    one96 = G.workspace_size(prob(**wide, tuning=G.Tuning(segment_tokens=4096, chain_group=1)), "bidir")
    on96 = G.workspace_size(prob(**wide, tuning=G.Tuning(segment_tokens=512, chain_group=1)), "bidir")
    assert on96 - one96 == pytest.approx(2 * 7 * 2 * 96 * (192 + 96) * 4, abs=1024)


def test_step_noalloc_rejects_oversized_steps_before_any_hip_call():
    """gdn_step_noalloc sizes the step on the host: one frame whose workspace
    exceeds the static scratch returns WORKSPACE_TOO_SMALL with nothing
    enqueued (fake pointers, no GPU); frames != 1 and a NULL state_out are
    argument errors as for gdn_step."""
    L = G.lib()
    vp = ctypes.c_void_p
    big = prob(batch=8, heads=64, d_k=112, d_v=112, frames=1, tokens_per_frame=60000, algo="chunked")
    assert G.workspace_size(big, "fwd") > G.NOALLOC_SCRATCH_BYTES
    args = [vp(FAKE)] * 5
    assert L.gdn_step_noalloc(ctypes.byref(big), *args, None, vp(FAKE), vp(FAKE), None) \
        == G.ERR_WORKSPACE_TOO_SMALL
    assert "static scratch" in L.gdn_last_error_message().decode()
    two = prob(frames=2, algo="chunked")
    assert L.gdn_step_noalloc(ctypes.byref(two), *args, None, vp(FAKE), vp(FAKE), None) == G.ERR_INVALID_ARGUMENT
    one = prob(frames=1, algo="chunked")
    assert L.gdn_step_noalloc(ctypes.byref(one), *args, None, None, vp(FAKE), None) == G.ERR_INVALID_ARGUMENT
    # one 880-token frame of 20 heads x 112 fits
    frame = prob(heads=20, d_k=112, d_v=112, frames=1, tokens_per_frame=880, algo="chunked")
    assert 0 < G.workspace_size(frame, "fwd") <= G.NOALLOC_SCRATCH_BYTES


def test_strip_scan_plan_and_workspace():
    """Forward- and backward-only calls of the chunked path with at most 32
    sub-chunks per head (T <= 2048) and no prologue take the strip scan: one
    segment of the whole (rounded) sequence and a workspace of 11008 bytes per
    sub-chunk and head (fp16 Tm diag(beta) and P, 5120 bytes each, and three
    rows of 64 fp32 gate factors); NO_STRIP_SCAN, longer calls, two-scan calls
    and the prologue keep segment maps."""
    sub = 2 * 5120 + 3 * 64 * 4
    for T, heads, d in ((300, 2, 64), (880, 20, 112), (2048, 3, 16), (1, 1, 32)):
        kw = dict(batch=2, heads=heads, d_k=d, d_v=d, frames=1, tokens_per_frame=T, qkv_dtype=G.BF16, algo="chunked")
        p = G.make_problem(**kw)
        U = (T + 63) // 64
        for direction in ("fwd", "bwd"):
            assert G.segment_plan(p, direction) == 64 * U
            assert G.workspace_size(p, direction) == (2 * heads * U * sub + 255) // 256 * 256
        with G.tuning(no_strip_scan=True):
            q = G.make_problem(**kw)
        assert G.workspace_size(q, "fwd") != G.workspace_size(p, "fwd")
    # just past the limit, and the other cases, keep segment maps
    p = G.make_problem(batch=1, heads=2, d_k=64, d_v=64, frames=1, tokens_per_frame=2049, qkv_dtype=G.BF16,
                       algo="chunked")
    assert G.segment_plan(p, "fwd") < 2049
    for kw, d in ((dict(), "bidir"), (dict(), "chunk_causal"), (dict(prologue="features"), "fwd")):
        p = G.make_problem(batch=1, heads=2, d_k=64, d_v=64, frames=4, tokens_per_frame=300, qkv_dtype=G.BF16,
                           algo="chunked", first_chunk_frames=1, chunk_frames=1, **kw)
        assert G.segment_plan(p, d) < 1200
