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
    assert L.gdn_abi_version() == G.ABI_VERSION == 1
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
    ("abi_version", 2), ("batch", 0), ("heads", -1), ("frames", 0), ("tokens_per_frame", 0),
    ("d_k", 20), ("d_k", 144), ("d_v", 8), ("qkv_dtype", 7), ("out_dtype", -1), ("algo", 9),
])
def test_bad_problem_fields_are_rejected(field, value):
    p = prob()
    setattr(p, field, value)
    with pytest.raises(G.GdnError) as e:
        G.workspace_size(p, "bidir")
    assert e.value.status == G.ERR_INVALID_ARGUMENT
    assert G.lib().gdn_last_error_message().decode() != ""


def test_reserved_and_key_scale_and_direction_checks():
    p = prob()
    p.reserved[0] = 1
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
            a = G.workspace_size(prob(**kw), d)
            b = G.workspace_size(prob(prologue="features", **kw), d)
            assert b - a in (fac, rounded), (kw, d, a, b)
    p = prob(prologue="features", first_chunk_frames=2, chunk_frames=1)
    assert G.workspace_size(p, "chunk_causal") > G.workspace_size(prob(first_chunk_frames=2, chunk_frames=1),
                                                                  "chunk_causal")


def test_split_chain_workspace():
    """A split chain adds group maps and group start states to the workspace;
    the knob is process-wide and restored."""
    p = prob(frames=40, tokens_per_frame=100, algo="chunked")
    try:
        G.set_segment_tokens(64)
        G.set_chain_group(1)
        whole = G.workspace_size(p, "fwd")
        G.set_chain_group(4)
        split = G.workspace_size(p, "fwd")
        bidir = G.workspace_size(p, "bidir")
        G.set_chain_group(1)
        assert bidir == G.workspace_size(p, "bidir")   # bidirectional chains are never split
    finally:
        G.set_chain_group(0)
        G.set_segment_tokens(0)
    steps = (40 * 100 + 63) // 64 - 1
    groups = (steps + 3) // 4
    extra = 1 * 2 * groups * 64 * (128 + 64) * 4
    assert split - whole == pytest.approx(extra, abs=512)


def test_inverse_reuse_workspace():
    """A forward-only chunked call with more than one segment holds 5 KB of
    fp16 inverse blocks per 64-token sub-chunk and head, whether or not their
    reuse is switched on; a bidirectional call holds none."""
    p = prob(frames=40, tokens_per_frame=100, algo="chunked")   # 4000 tokens: 63 sub-chunks
    try:
        G.set_chain_group(1)
        G.set_segment_tokens(4096)      # one segment: no maps, no inverse blocks
        one = G.workspace_size(p, "fwd")
        one_bi = G.workspace_size(p, "bidir")
        G.set_segment_tokens(512)       # 8 segments
        on = G.workspace_size(p, "fwd")
        on_bi = G.workspace_size(p, "bidir")
        G.set_inverse_reuse(False)
        assert G.workspace_size(p, "fwd") == on
    finally:
        G.set_inverse_reuse(True)
        G.set_chain_group(0)
        G.set_segment_tokens(0)
    per_seg = 2 * 64 * (128 + 64) * 4           # one scan's map and start state, 2 heads
    tm = 2 * 63 * 5120
    assert on - one == pytest.approx(7 * per_seg + tm, abs=1024)
    assert on_bi - one_bi == pytest.approx(2 * 7 * per_seg, abs=1024)
