"""Python binding of libgdn (frame-wise gated delta rule layer forward, gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libgdn.so``.  PyTorch supplies device memory and the current HIP
stream.  The names mirror the C ABI in ``include/gdn.h``: ``forward`` wraps
``gdn_forward``, ``step`` wraps ``gdn_step``, ``workspace_size`` wraps
``gdn_workspace_size``.

There is no CPU fallback: if the library is not built, or a call is made with
tensors that are not on a GPU, these functions raise.
"""
from __future__ import annotations

import contextlib
import contextvars
import ctypes
import dataclasses
import os

__all__ = ["forward", "step", "step_noalloc", "workspace_size", "NOALLOC_SCRATCH_BYTES", "make_problem", "lib", "GdnError", "Tuning", "tuning",
           "segment_plan", "profile_enable", "profile_reset", "profile_read",
           "FORWARD", "BACKWARD", "BIDIRECTIONAL", "CHUNK_CAUSAL", "ABI_VERSION", "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn.so")
ABI_VERSION = 2

OK, ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, ERR_WORKSPACE_TOO_SMALL, ERR_HIP = range(5)
F32, BF16 = 0, 1
FORWARD, BACKWARD, BIDIRECTIONAL, CHUNK_CAUSAL = 0, 1, 2, 3
ALGO = {"auto": 0, "chunked": 1, "recurrent": 2}
INTRA = {"sequential": 0, "jacobi": 1}
PROLOGUE = {"none": 0, "features": 1}
FLAG_SERIAL_SCANS, FLAG_FORM_INVERSE, FLAG_NO_STRIP_SCAN = 1, 2, 4
NOALLOC_SCRATCH_BYTES = 64 << 20   # GDN_NOALLOC_SCRATCH_BYTES
DIRECTION = {"fwd": FORWARD, "bwd": BACKWARD, "bidir": BIDIRECTIONAL, "chunk_causal": CHUNK_CAUSAL,
             FORWARD: FORWARD, BACKWARD: BACKWARD, BIDIRECTIONAL: BIDIRECTIONAL, CHUNK_CAUSAL: CHUNK_CAUSAL}


class GdnError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} [status {status}]")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("frames", ctypes.c_int32), ("tokens_per_frame", ctypes.c_int32),
                ("qkv_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("algo", ctypes.c_int32), ("key_scale", ctypes.c_float),
                ("intra", ctypes.c_int32), ("first_chunk_frames", ctypes.c_int32),
                ("chunk_frames", ctypes.c_int32), ("prologue", ctypes.c_int32),
                ("segment_tokens", ctypes.c_int32), ("chain_group", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("reserved", ctypes.c_int32 * 5)]


@dataclasses.dataclass(frozen=True)
class Tuning:
    """Tuning fields of a call's problem (gdn.h, gdn_problem): they change the
    plan of the chunked and frame-level paths, never the results beyond
    rounding.  segment_tokens: tokens per segment (0 = automatic);
    chain_group: 0 automatic, 1 whole chain, m >= 2 groups of m maps;
    serial_scans: run a two-scan call's kernels in order on the caller's
    stream; form_inverse: the output kernel of a single-scan call forms its
    sub-chunk inverses instead of loading the map kernel's; no_strip_scan:
    a short single-scan call (T <= 2048) runs through segment maps and their
    chain instead of the strip scan."""

    segment_tokens: int = 0
    chain_group: int = 0
    serial_scans: bool = False
    form_inverse: bool = False
    no_strip_scan: bool = False


_TUNING = contextvars.ContextVar("gdn_tuning", default=Tuning())


@contextlib.contextmanager
def tuning(**fields):
    """Context in which calls without an explicit ``tuning`` argument use these
    Tuning fields (per thread / task; the library itself keeps no such state)."""
    tok = _TUNING.set(dataclasses.replace(_TUNING.get(), **fields))
    try:
        yield
    finally:
        _TUNING.reset(tok)


_lib = None


def lib():
    """The loaded libgdn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libgdn.so is not built ({LIB_PATH}); run "
                              "`python -m gated_delta_rule_frame_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
        P = ctypes.POINTER(Problem)
        L.gdn_abi_version.restype = i32
        L.gdn_abi_version.argtypes = []
        L.gdn_status_string.restype = ctypes.c_char_p
        L.gdn_status_string.argtypes = [i32]
        L.gdn_last_error_message.restype = ctypes.c_char_p
        L.gdn_last_error_message.argtypes = []
        L.gdn_workspace_size.restype = i32
        L.gdn_workspace_size.argtypes = [P, i32, ctypes.POINTER(sz)]
        L.gdn_forward.restype = i32
        L.gdn_forward.argtypes = [P, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.gdn_profile_enable.restype = i32
        L.gdn_profile_enable.argtypes = [i32]
        L.gdn_profile_reset.restype = i32
        L.gdn_profile_reset.argtypes = []
        L.gdn_profile_read.restype = i32
        L.gdn_profile_read.argtypes = [i32, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double)]
        L.gdn_kernel_name.restype = ctypes.c_char_p
        L.gdn_kernel_name.argtypes = [i32]
        L.gdn_plan_segment_tokens.restype = i32
        L.gdn_plan_segment_tokens.argtypes = [P, i32, ctypes.POINTER(i32)]
        L.gdn_step.restype = i32
        L.gdn_step.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.gdn_step_noalloc.restype = i32
        L.gdn_step_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        if L.gdn_abi_version() != ABI_VERSION:
            raise ImportError(f"libgdn ABI {L.gdn_abi_version()} != binding ABI {ABI_VERSION}")
        _lib = L
    return _lib


def _check(status):
    if status != OK:
        L = lib()
        raise GdnError(status, f"{L.gdn_status_string(status).decode()}: "
                               f"{L.gdn_last_error_message().decode()}")


def make_problem(batch, heads, d_k, d_v, frames, tokens_per_frame, qkv_dtype=BF16,
                 out_dtype=BF16, algo="auto", key_scale=1.0, intra="sequential", first_chunk_frames=0,
                 chunk_frames=0, prologue="none", tuning=None):
    """A gdn_problem; ``tuning`` (a Tuning) defaults to the current tuning context."""
    t = _TUNING.get() if tuning is None else tuning
    p = Problem()
    p.abi_version = ABI_VERSION
    p.batch, p.heads, p.d_k, p.d_v = batch, heads, d_k, d_v
    p.frames, p.tokens_per_frame = frames, tokens_per_frame
    p.qkv_dtype, p.out_dtype = qkv_dtype, out_dtype
    p.algo = ALGO[algo] if isinstance(algo, str) else int(algo)
    p.key_scale = float(key_scale)
    p.intra = INTRA[intra] if isinstance(intra, str) else int(intra)
    p.first_chunk_frames, p.chunk_frames = int(first_chunk_frames), int(chunk_frames)
    p.prologue = PROLOGUE[prologue] if isinstance(prologue, str) else int(prologue)
    p.segment_tokens, p.chain_group = int(t.segment_tokens), int(t.chain_group)
    p.flags = (FLAG_SERIAL_SCANS if t.serial_scans else 0) | (FLAG_FORM_INVERSE if t.form_inverse else 0) | \
        (FLAG_NO_STRIP_SCAN if t.no_strip_scan else 0)
    return p


def workspace_size(problem: Problem, direction=BIDIRECTIONAL) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().gdn_workspace_size(ctypes.byref(problem), DIRECTION[direction], ctypes.byref(n)))
    return n.value


KERNELS = ("seg_map_kernel", "seg_chain_kernel", "seg_out_kernel", "recurrent_kernel", "jac_map_kernel",
           "jac_out_kernel", "prologue_kernel", "scan_prep_kernel", "scan_kernel")


def profile_enable(on: bool = True) -> None:
    """Bracket every libgdn kernel launch with HIP events (see gdn.h)."""
    _check(lib().gdn_profile_enable(1 if on else 0))


def profile_reset() -> None:
    _check(lib().gdn_profile_reset())


def profile_read() -> dict:
    """{kernel name: (launches, total ms)} since the last reset; waits for the events."""
    out = {}
    for i, name in enumerate(KERNELS):
        n, ms = ctypes.c_int64(0), ctypes.c_double(0.0)
        _check(lib().gdn_profile_read(i, ctypes.byref(n), ctypes.byref(ms)))
        out[name] = (n.value, ms.value)
    return out


def segment_plan(problem: Problem, direction=BIDIRECTIONAL) -> int:
    """Tokens per segment the chunked path uses (0 = token-recurrent path)."""
    n = ctypes.c_int32(0)
    _check(lib().gdn_plan_segment_tokens(ctypes.byref(problem), DIRECTION[direction], ctypes.byref(n)))
    return n.value


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _prepare(q, k, v, log_gate, beta, frames, tokens_per_frame, out, out_dtype, algo, key_scale,
             intra="sequential", chunks=(0, 0), prologue="none", tuning=None):
    """Checks the inputs (and a caller-supplied ``out``) and builds the problem.
    The output dtype is ``out_dtype``, else that of ``out``, else fp32."""
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v), ("log_gate", log_gate), ("beta", beta)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a tensor on a GPU")
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k must be [B,T,H,d_k] and v [B,T,H,d_v]")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    B, T, H, dk = q.shape
    dv = v.shape[3]
    if log_gate.shape != (B, T, H) or beta.shape != (B, T, H):
        raise ValueError("log_gate and beta must be [B,T,H]")
    if log_gate.dtype != torch.float32 or beta.dtype != torch.float32:
        raise TypeError("log_gate and beta must be float32")
    if tokens_per_frame is None:
        tokens_per_frame = T if frames is None else T // frames
    if frames is None:
        frames = T // tokens_per_frame
    if frames * tokens_per_frame != T:
        raise ValueError(f"frames * tokens_per_frame = {frames * tokens_per_frame} != T = {T}")
    if out is not None:
        if not isinstance(out, torch.Tensor) or out.device != q.device or not out.is_contiguous() \
                or tuple(out.shape) != (B, T, H, dv) or out.dtype not in (torch.float32, torch.bfloat16):
            raise ValueError(f"out must be a contiguous float32 or bfloat16 tensor of shape "
                             f"{(B, T, H, dv)} on {q.device}")
        if out_dtype is not None and out_dtype != out.dtype:
            raise TypeError(f"out_dtype {out_dtype} differs from out's dtype {out.dtype}")
        odt = out.dtype
    else:
        odt = torch.float32 if out_dtype is None else out_dtype
    p = make_problem(B, H, dk, dv, frames, tokens_per_frame, _dtype_code(q),
                     _dtype_code(torch.empty(0, dtype=odt)), algo, key_scale, intra, *chunks, prologue,
                     tuning=tuning)
    return p, (B, T, H, dk, dv), odt


def _state_tensor(t, shape, name, device):
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device != device or t.dtype != torch.float32 \
            or not t.is_contiguous() or tuple(t.shape) != shape:
        raise ValueError(f"{name} must be a contiguous float32 tensor of shape {shape} on {device}")
    return t


def _workspace(problem, direction, workspace, device):
    torch = _torch()
    need = workspace_size(problem, direction)
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or workspace.device != device or not workspace.is_contiguous():
            raise ValueError(f"workspace must be a contiguous tensor on {device}")
        return workspace, workspace.numel() * workspace.element_size()
    if need == 0:
        return None, 0
    return torch.empty(need, dtype=torch.uint8, device=device), need


def forward(q, k, v, log_gate, beta, initial_state=None, direction="bidir", *, frames=None,
            tokens_per_frame=None, key_scale=1.0, out_dtype=None, algo="auto",
            out=None, final_state=None, want_state=True, workspace=None, intra="sequential",
            first_chunk_frames=0, chunk_frames=0, prologue="none", tuning=None):
    """Whole-sequence layer forward (gdn_forward); returns (out, final_state).

    q, k: [B,T,H,d_k]; v: [B,T,H,d_v] (fp32 or bf16, one dtype); log_gate,
    beta: [B,T,H] fp32; initial_state: [B,H,d_k,d_v] fp32 or None (zeros).
    The output is fp32 unless ``out_dtype`` (or a supplied ``out``) says
    otherwise (a bf16 output adds a rounding of up to 2^-8 |o| per element).  ``intra="jacobi"`` selects the
    frame-level transition; ``direction="chunk_causal"`` with
    ``first_chunk_frames`` / ``chunk_frames`` the chunk-causal layer;
    ``prologue="features"`` applies the key features ReLU(RMSNorm(k)) and the
    query normalisation on load (see gdn.h).  ``tuning`` (a Tuning) defaults
    to the current ``tuning()`` context.
    """
    torch = _torch()
    p, (B, T, H, dk, dv), odt = _prepare(q, k, v, log_gate, beta, frames, tokens_per_frame, out,
                                         out_dtype, algo, key_scale, intra,
                                         (first_chunk_frames, chunk_frames), prologue, tuning)
    d = DIRECTION[direction]
    shape = (B, H, dk, dv)
    initial_state = _state_tensor(initial_state, shape, "initial_state", q.device)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=odt, device=q.device)
    if final_state is None and want_state:
        final_state = torch.empty(shape, dtype=torch.float32, device=q.device)
    final_state = _state_tensor(final_state, shape, "final_state", q.device)
    ws, ws_bytes = _workspace(p, d, workspace, q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(lib().gdn_forward(ctypes.byref(p), d, _ptr(q), _ptr(k), _ptr(v), _ptr(log_gate),
                             _ptr(beta), _ptr(initial_state), _ptr(out), _ptr(final_state),
                             _ptr(ws), ws_bytes, ctypes.c_void_p(stream)))
    return out, final_state


def step(q, k, v, log_gate, beta, state_in=None, state_out=None, *, key_scale=1.0,
         out_dtype=None, algo="auto", out=None, workspace=None, intra="sequential", prologue="none",
         tuning=None):
    """One frame of the chunk-causal forward scan (gdn_step); returns (out, state_out).

    The inputs hold exactly one frame ([B,S,H,d]); state_out may be state_in.
    """
    torch = _torch()
    p, (B, T, H, dk, dv), odt = _prepare(q, k, v, log_gate, beta, 1, None, out, out_dtype, algo,
                                         key_scale, intra, (0, 0), prologue, tuning)
    shape = (B, H, dk, dv)
    state_in = _state_tensor(state_in, shape, "state_in", q.device)
    if state_out is None:
        state_out = torch.empty(shape, dtype=torch.float32, device=q.device)
    state_out = _state_tensor(state_out, shape, "state_out", q.device)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=odt, device=q.device)
    ws, ws_bytes = _workspace(p, FORWARD, workspace, q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(lib().gdn_step(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(log_gate), _ptr(beta),
                          _ptr(state_in), _ptr(state_out), _ptr(out), _ptr(ws), ws_bytes,
                          ctypes.c_void_p(stream)))
    return out, state_out


def step_noalloc(q, k, v, log_gate, beta, state_in=None, state_out=None, *, key_scale=1.0,
                 out_dtype=None, algo="auto", out=None, intra="sequential", prologue="none", tuning=None):
    """gdn_step_noalloc: one frame like ``step`` with the library's static device
    scratch in place of a workspace; returns (out, state_out).  The library
    allocates nothing; pass ``out`` and ``state_out`` to keep this call free of
    torch allocations too."""
    torch = _torch()
    p, (B, T, H, dk, dv), odt = _prepare(q, k, v, log_gate, beta, 1, None, out, out_dtype, algo,
                                         key_scale, intra, (0, 0), prologue, tuning)
    shape = (B, H, dk, dv)
    state_in = _state_tensor(state_in, shape, "state_in", q.device)
    if state_out is None:
        state_out = torch.empty(shape, dtype=torch.float32, device=q.device)
    state_out = _state_tensor(state_out, shape, "state_out", q.device)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=odt, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(lib().gdn_step_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(log_gate), _ptr(beta),
                                  _ptr(state_in), _ptr(state_out), _ptr(out), ctypes.c_void_p(stream)))
    return out, state_out
