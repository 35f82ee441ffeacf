#!/usr/bin/env python3
"""One-GPU benchmark of the frame-wise gated delta rule layer forward.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--direction D]

A step is one whole-sequence layer forward (gdn_forward) over one batch of
synthetic inputs already resident in HBM.  The default workload is the 60 s
720p clip: batch 1, 20 heads x 112, 121 latent frames x 880 tokens (106,480
tokens), bf16 q/k/v, fp32 gates/state/accumulation and fp32 output, run in
bidirectional mode (forward scan + reversed scan, summed), as in the SANA-WM
summary page, section 3.2 "Bidirectional and Chunk-Causal GDN Variants".
With ``--workload stream60s_121x880_h20d112`` a step is the chunk-causal
streaming loop: 121 gdn_step calls of one 880-token frame each, the state
carried in place.

Before timing, the outputs and final states of every (batch, head) pair are
checked against the float64 CPU oracle over the whole sequence (heads are
independent, so a head's outputs and final state are exact targets; 16 worker
processes of one thread each); that same oracle run, and one pair on one
thread, are the reported CPU baseline.  The default run also measures, as
secondary figures in the same line, the forward-only scan of the clip, the 5 s
clip, the batched 2 x 35 x 64 workload (bidirectional and forward-only) and
the 121-call streaming loop (per call, whole loop, and the loop replayed as
one HIP graph), each checked on one (batch, head) pair.  Prints exactly one
JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import dataclasses
import hashlib
import json
import os
import platform
import re
import shutil
import sys
import tempfile
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN layer fwd tokens/s & % bf16 MFMA peak, 121×880-token 60 s clip, 1 GPU"
FLOP_PER_CLK_CU = 4096      # dense fp16/bf16 MFMA flops per clock per compute unit (CDNA4)
NOMINAL_CUS, NOMINAL_MHZ = 256, 2400
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TOL = {"f32": 1e-4, "bf16": 2e-2}
KERNEL_SOURCES = ("gdn_chunked.hip", "gdn_prologue.hip", "gdn_mfma.h", "gdn_common.h")
SUB = 64                    # tokens per sub-chunk of the chunked path


# ---------------------------------------------------------------- peak

def device_peak():
    """(compute units, shader clock MHz, dense fp16/bf16 MFMA peak TFLOP/s, source)
    read from the HIP runtime of device 0 (hipDeviceGetAttribute); the
    nominal MI355X figures if the runtime cannot be queried."""
    cands = []
    try:
        import torch
        cands.append(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
    except Exception:
        pass
    cands += [os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib", "libamdhip64.so"), "libamdhip64.so"]
    for c in cands:
        try:
            hip = ctypes.CDLL(c)
        except OSError:
            continue
        cu, clk = ctypes.c_int(0), ctypes.c_int(0)
        # hipDeviceAttributeMultiprocessorCount = 63, hipDeviceAttributeClockRate = 5 (kHz)
        if hip.hipDeviceGetAttribute(ctypes.byref(cu), 63, 0) == 0 and \
                hip.hipDeviceGetAttribute(ctypes.byref(clk), 5, 0) == 0 and cu.value > 0 and clk.value > 0:
            mhz = clk.value / 1e3
            return cu.value, mhz, cu.value * FLOP_PER_CLK_CU * mhz * 1e6 / 1e12, "hipDeviceGetAttribute"
    return NOMINAL_CUS, NOMINAL_MHZ, NOMINAL_CUS * FLOP_PER_CLK_CU * NOMINAL_MHZ * 1e6 / 1e12, "nominal"


# ---------------------------------------------------------------- FLOP models

def canonical_flops(C, dk, dv):
    """Chunk count per (batch, head, chunk of C tokens, direction): strict-lower
    K K^T plus forward substitution on [W|U], causal Q K^T and its product with
    U', and the three C x d x d state products (W H, Q H, K^T U')."""
    return C * (C - 1) * (2 * dk + dv) + C * (C + 1) * (dk + dv) + 6 * C * dk * dv


def subchunk_sizes(T, L, c=SUB):
    """Token counts of the 64-token sub-chunks, per segment of L tokens."""
    return [[min(c, min(L, T - s0) - a) for a in range(0, min(L, T - s0), c)] for s0 in range(0, T, L)]


def chunk_subchunks(T, S, first, every, c=SUB):
    """Sub-chunk sizes of the chunk-causal reversed scan (each chunk of frames cut from its start)."""
    out, t0, n = [], 0, first * S
    while t0 < T:
        t1 = min(T, t0 + n)
        out.append([min(c, t1 - a) for a in range(t0, t1, c)])
        t0, n = t1, every * S
    return out


def own_flops(segs, dk, dv):
    """The method's own work on the executed sub-chunks: the canonical count at
    each sub-chunk's size n (summed), per (batch, head) and direction."""
    return sum(canonical_flops(n, dk, dv) for seg in segs for n in seg)


def map_term(segs, dk):
    """The extra work of forming the transition part of a segment map, 2 n d_k^2
    per sub-chunk (the prefix composition of transition maps)."""
    return sum(2 * n * dk * dk for seg in segs for n in seg)


def out_alg_flops(n, dk, dv):
    """Credited work of the output kernel on one sub-chunk: the canonical count
    without the W substitution (n(n-1) d_k), which the correction form never
    forms, capped by what the kernel executes apart from the explicit inverse."""
    canon = canonical_flops(n, dk, dv) - n * (n - 1) * dk
    executed = n * (n - 1) * dk + 3 * n * (n + 1) * dv + 6 * n * dk * dv
    return min(canon, executed)


def out_flops(n, d, inverse=True):
    """Executed flops of the output pass on one sub-chunk of n tokens: causal
    Q K^T, K H and Q H, Tm diag(beta) R and P V' (triangular), the state update,
    and (inverse: unless it loads the map kernel's) the strict-lower K K^T and
    the triangular inverse (n^3/3)."""
    tri = n * (n - 1) * d + n ** 3 // 3 if inverse else 0
    return tri + 3 * n * (n + 1) * d + 6 * n * d * d


def map_flops(n, d, q_only=False):
    """Executed flops of the segment-map pass on one sub-chunk (state [P|Q], 2d
    columns; q_only: Q alone, d columns)."""
    w = 1 if q_only else 2
    return n * (n - 1) * d + w * n * (n + 1) * d + 4 * w * n * d * d + n ** 3 // 3


def executed_flops(T, L, d, bh, ndir, reuse=True):
    """Executed flops per call of each chunked-path kernel (diagnostic)."""
    segs = subchunk_sizes(T, L)
    reuse = reuse and len(segs) > 1 and ndir == 1
    per_out = sum(out_flops(n, d, inverse=not reuse) for seg in segs for n in seg)
    if ndir == 1:
        maps = sum(map_flops(n, d) for seg in (segs if reuse else segs[:-1]) for n in seg)
    else:
        maps = sum(map_flops(n, d) for seg in segs for n in seg)
        maps += sum(map_flops(n, d, q_only=True) for seg in segs[1:] for n in seg)
    chain = (len(segs) - 1) * 2 * d ** 3
    return {"seg_out_kernel": per_out * bh * ndir, "seg_map_kernel": maps * bh,
            "seg_chain_kernel": chain * bh * ndir}


def jacobi_flops(S, F, d, bh, ndir):
    """Per-call flops of the frame-level path, per kernel: per frame
    c^2 K^T diag(beta) K and c K^T diag(beta) V (4 S d^2), the outputs Q H_end
    (2 S d^2), and one d x d state product per frame and scan (2 d^3)."""
    return {"jac_map_kernel": 4 * S * d * d * F * bh, "jac_out_kernel": 2 * S * d * d * F * bh,
            "seg_chain_kernel": 2 * d ** 3 * F * bh * ndir}


def jacobi_bytes(S, F, d, bh, ndir, out_bytes=4):
    """Algorithmic HBM bytes per call of the frame-level path, per kernel."""
    T = S * F
    maps = ndir * F * bh * d * 2 * d * 4
    states = ndir * (F + 1) * bh * d * d * 4
    return {"jac_map_kernel": T * bh * (2 * d * 2 + 4) + maps,
            "jac_out_kernel": T * bh * (2 * d + out_bytes * d) + states,
            "seg_chain_kernel": maps + states}


def algorithmic_bytes(B, T, H, dk, dv, qkv_bytes=2, out_bytes=4, state=True):
    """q, k, v read once, gates and beta read once, the output written once,
    the state read and written once."""
    return B * T * H * ((2 * dk + dv) * qkv_bytes + 8 + dv * out_bytes) + (2 * B * H * dk * dv * 4 if state else 0)


# ---------------------------------------------------------------- counters

def kernel_source_hash():
    """Hash of the kernel sources without their // comments and with runs of
    whitespace collapsed: a change of wording alone keeps the counters valid."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "gated_delta_rule_frame_amd", "csrc", f)) as fh:
            code = re.sub(r"//[^\n]*", "", fh.read())
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def read_traffic(kernel, tag):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if it is missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{tag}_counters.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except OSError:
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


# ---------------------------------------------------------------- oracle (CPU baseline leg)

def _oracle_head(spec):
    """One (batch, head) of the oracle over the whole sequence, in a worker
    process: inputs memory-mapped from the run's scratch folder.  Returns
    (index, out, final state, seconds)."""
    from threadpoolctl import threadpool_limits
    from oracle import gdn_oracle as O
    folder, i, b, h, kind, key_scale, S, chunks = spec
    # the arrays are stored head-major ([B, H, T, ...]): one head is contiguous
    a = [np.ascontiguousarray(np.load(os.path.join(folder, f"{n}.npy"), mmap_mode="r")[b, h])[None, :, None]
         for n in ("q", "k", "v", "log_gate", "beta")]
    h0 = np.load(os.path.join(folder, "h0.npy"), mmap_mode="r")[b:b + 1, h:h + 1]
    with threadpool_limits(1):
        t0 = time.perf_counter()
        ro, rH = run_oracle(O, kind, a, np.ascontiguousarray(h0), key_scale, S, chunks)
        dt = time.perf_counter() - t0
    return i, ro, rH, dt


def run_oracle(O, kind, a, h0, key_scale, S, chunks):
    """kind: (direction, intra, prologue)."""
    direction, intra, pro = kind
    a = list(a)
    if pro:
        a[0], a[1] = O.query_features(a[0]), O.key_features(a[1])
    if intra == "jacobi":
        return O.jacobi_forward(direction, *a, h0, key_scale=key_scale, tokens_per_frame=S)
    if direction == "chunk_causal":
        return O.chunk_causal(*a, h0, key_scale=key_scale, tokens_per_frame=S,
                              first_chunk_frames=chunks[0], chunk_frames=chunks[1])
    return O.forward(direction, *a, h0, key_scale=key_scale)


def oracle_pool(x, pairs, kind, key_scale, S, chunks, procs):
    """The oracle on (batch, head) pairs in a pool of `procs` spawned
    processes (one thread each).  Returns ({pair: (out, state)}, wall seconds,
    summed per-head seconds)."""
    import multiprocessing as mp
    folder = tempfile.mkdtemp(prefix="gdn_bench_", dir="/dev/shm" if os.path.isdir("/dev/shm") else None)
    try:
        for n in ("q", "k", "v", "log_gate", "beta"):
            np.save(os.path.join(folder, f"{n}.npy"), np.ascontiguousarray(np.swapaxes(x[n], 1, 2)))
        np.save(os.path.join(folder, "h0.npy"), x["h0"])
        specs = [(folder, i, b, h, kind, key_scale, S, chunks) for i, (b, h) in enumerate(pairs)]
        ctx = mp.get_context("spawn")
        t0 = time.perf_counter()
        with ctx.Pool(procs) as pool:
            res = pool.map(_oracle_head, specs, chunksize=1)
        wall = time.perf_counter() - t0
    finally:
        shutil.rmtree(folder, ignore_errors=True)
    return {pairs[i]: (ro, rH) for i, ro, rH, _ in res}, wall, sum(r[3] for r in res)


def rel(u, r):
    return float(np.max(np.abs(u - r)) / np.sqrt(np.mean(r * r)))


# ---------------------------------------------------------------- GPU harness

class Run:
    """One workload and call configuration on the GPU: inputs resident in HBM,
    preallocated outputs and workspace, a step() that enqueues one layer forward."""

    def __init__(self, G, torch, w, direction, seed=0, intra="sequential", prologue="none",
                 chunks=(4, 3), tuning=None):
        from gdn_inputs import make_inputs
        self.G, self.torch, self.w = G, torch, w
        self.direction, self.intra, self.prologue, self.chunks = direction, intra, prologue, chunks
        self.tuning = tuning or G.Tuning()
        dev = torch.device("cuda:0")
        self.x = x = make_inputs(w, seed)
        qkv_dt = torch.bfloat16 if w.qkv_dtype == "bf16" else torch.float32
        self.d = {n: torch.from_numpy(x[n]).to(dev, qkv_dt) for n in ("q", "k", "v")}
        for n in ("log_gate", "beta"):
            self.d[n] = torch.from_numpy(x[n]).to(dev)
        self.h0 = torch.from_numpy(x["h0"]).to(dev) if np.any(x["h0"]) else None
        B, T, H, dk, dv = w.batch, w.tokens, w.heads, w.d_k, w.d_v
        pro, jac = prologue == "features", intra == "jacobi"
        self.key_scale = (dk * w.tokens_per_frame) ** -0.5 if pro else w.tokens_per_frame ** -0.5 if jac else 1.0
        self.stream_mode = direction == "stream"
        S = w.tokens_per_frame
        self.prob = G.make_problem(B, H, dk, dv, 1 if self.stream_mode else w.frames, S,
                                   G.BF16 if w.qkv_dtype == "bf16" else G.F32, G.F32, "auto", self.key_scale,
                                   intra, chunks[0], chunks[1], prologue, tuning=self.tuning)
        pdir = "fwd" if self.stream_mode else direction
        self.L = G.segment_plan(self.prob, pdir)
        self.ws = torch.empty(max(G.workspace_size(self.prob, pdir), 16), dtype=torch.uint8, device=dev)
        self.out = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
        self.hT = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
        if self.stream_mode:
            if B != 1:
                raise ValueError("the streaming loop slices frames of a batch-1 sequence in place")
            self.frames = [{n: self.d[n][:, f * S:(f + 1) * S] for n in ("q", "k", "v", "log_gate", "beta")}
                           for f in range(w.frames)]
            self.outs = [self.out[:, f * S:(f + 1) * S] for f in range(w.frames)]

    def call(self, f):
        """One gdn_step call of the streaming loop (frame f, state in place)."""
        fr = self.frames[f]
        self.G.step(fr["q"], fr["k"], fr["v"], fr["log_gate"], fr["beta"], self.hT, self.hT,
                    key_scale=self.key_scale, out=self.outs[f], workspace=self.ws, prologue=self.prologue,
                    tuning=self.tuning)

    def step(self, tuning=None):
        if self.stream_mode:
            if self.h0 is None:
                self.hT.zero_()
            else:
                self.hT.copy_(self.h0)
            for f in range(self.w.frames):
                self.call(f)
            return
        d = self.d
        self.G.forward(d["q"], d["k"], d["v"], d["log_gate"], d["beta"], self.h0, self.direction,
                       tokens_per_frame=self.w.tokens_per_frame, out=self.out, final_state=self.hT,
                       workspace=self.ws, key_scale=self.key_scale, intra=self.intra,
                       first_chunk_frames=self.chunks[0], chunk_frames=self.chunks[1], prologue=self.prologue,
                       tuning=tuning or self.tuning)

    def kind(self):
        return ("fwd" if self.stream_mode else self.direction, self.intra, self.prologue == "features")

    def parity(self, pairs, results):
        """Worst relative errors of out and final state over `pairs` against
        oracle results {pair: (out, state)}."""
        errs = {}
        for (b, h) in pairs:
            ro, rH = results[(b, h)]
            o = self.out[b:b + 1, :, h:h + 1].double().cpu().numpy()
            s = self.hT[b:b + 1, h:h + 1].double().cpu().numpy()
            errs[f"{b},{h}"] = [round(rel(o, ro), 6), round(rel(s, rH), 6)]
        eo = max(e[0] for e in errs.values())
        es = max(e[1] for e in errs.values())
        tol = TOL[self.w.qkv_dtype]
        return {"pairs": len(errs), "out_err": eo, "state_err": es, "tol": tol,
                "pass": eo <= tol and es <= tol, "per_head": errs}

    def oracle_local(self, pairs):
        """The oracle in this process, one thread (the single-core baseline)."""
        from threadpoolctl import threadpool_limits
        from oracle import gdn_oracle as O
        res, secs = {}, 0.0
        for (b, h) in pairs:
            a = [self.x[n][b:b + 1, :, h:h + 1] for n in ("q", "k", "v", "log_gate", "beta")]
            with threadpool_limits(1):
                t0 = time.perf_counter()
                res[(b, h)] = run_oracle(O, self.kind(), a, self.x["h0"][b:b + 1, h:h + 1], self.key_scale,
                                         self.w.tokens_per_frame, self.chunks)
                secs += time.perf_counter() - t0
        return res, secs


def time_steps(torch, run, steps, warmup, tuning=None):
    for _ in range(warmup):
        run.step(tuning)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        run.step(tuning)
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps


def stream_detail(torch, run, reps):
    """The 121-call loop: per-call durations (HIP events on the call's stream),
    and the loop captured once as a HIP graph and replayed."""
    F = run.w.frames
    per_call = []
    for _ in range(reps):
        run.hT.zero_()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(F + 1)]
        evs[0].record()
        for f in range(F):
            run.call(f)
            evs[f + 1].record()
        torch.cuda.synchronize()
        per_call += [evs[f].elapsed_time(evs[f + 1]) for f in range(F)]
    eager_out, eager_state = run.out.clone(), run.hT.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run.hT.zero_()
        for f in range(F):
            run.call(f)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run.hT.zero_()
        for f in range(F):
            run.call(f)
    torch.cuda.synchronize()
    ok = True
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        ok = ok and torch.equal(run.out, eager_out) and torch.equal(run.hT, eager_state)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    graph_ms = ev0.elapsed_time(ev1) / reps
    pc = np.array(per_call)
    return {"calls": F, "per_call_us_median": float(np.median(pc) * 1e3), "per_call_us_min": float(pc.min() * 1e3),
            "graph_loop_ms": graph_ms, "graph_per_call_us": graph_ms / F * 1e3, "graph_matches_eager": bool(ok)}


def flops_of(run, B, H, dk, dv, T, ndir):
    """(own GFLOP, own + map term GFLOP, per-kernel executed flops, credited
    flops per launch of the output kernel or None) per step."""
    w = run.w
    if run.intra == "jacobi":
        fl = jacobi_flops(w.tokens_per_frame, w.frames, dk, B * H, ndir)
        return sum(fl.values()), sum(fl.values()), fl, None
    if run.stream_mode:
        segs = subchunk_sizes(w.tokens_per_frame, run.L)
        calls = w.frames
        own = own_flops(segs, dk, dv) * B * H * calls
        mt = map_term(segs, dk) * B * H * calls
        fl = {k: v * calls for k, v in executed_flops(w.tokens_per_frame, run.L, dk, B * H, 1).items()}
        alg_out = sum(out_alg_flops(n, dk, dv) for s in segs for n in s) * B * H
        return own, own + mt, fl, alg_out
    segs = subchunk_sizes(T, run.L)
    if run.direction == "chunk_causal":
        rsegs = chunk_subchunks(T, w.tokens_per_frame, *run.chunks)
        own = (own_flops(segs, dk, dv) + own_flops(rsegs, dk, dv)) * B * H
        mt = map_term(segs, dk) * B * H
        fl = executed_flops(T, run.L, dk, B * H, 1, reuse=False)
        fl["seg_out_kernel"] += sum(out_flops(n, dk) for s in rsegs for n in s) * B * H
        alg_out = (sum(out_alg_flops(n, dk, dv) for s in segs for n in s) +
                   sum(out_alg_flops(n, dk, dv) for s in rsegs for n in s)) * B * H / 2
        return own, own + mt, fl, alg_out
    own = own_flops(segs, dk, dv) * B * H * ndir
    mt = map_term(segs, dk) * B * H * ndir
    fl = executed_flops(T, run.L, dk, B * H, ndir, reuse=not run.tuning.form_inverse)
    alg_out = sum(out_alg_flops(n, dk, dv) for s in segs for n in s) * B * H
    return own, own + mt, fl, alg_out


def measure(G, torch, run, steps, warmup, peak_tflops, tag):
    """Times `run` and returns its figures (no parity)."""
    w = run.w
    B, T, H, dk, dv = w.batch, w.tokens, w.heads, w.d_k, w.d_v
    ndir = 2 if run.direction in ("bidir", "chunk_causal") else 1
    ms = time_steps(torch, run, steps, warmup)
    # Per-kernel durations: HIP events recorded by the library on each
    # kernel's stream.  "kernels": each kernel alone (the in-order schedule of
    # the same call), the figures the roofline uses; "kernels_in_schedule":
    # in the timed schedule, where a two-scan call runs kernels of both scans
    # side by side and each duration includes the sharing.
    psteps = max(3, steps // 2)

    def kernel_times(tuning):
        G.profile_reset()
        G.profile_enable(True)
        time_steps(torch, run, psteps, 1, tuning)
        G.profile_enable(False)
        prof = G.profile_read()
        return {k: {"launches_per_step": n / (psteps + 1), "avg_ms": t / n} for k, (n, t) in prof.items() if n}

    shared = kernel_times(None)
    serial = dataclasses.replace(run.tuning, serial_scans=True)
    kern = kernel_times(serial) if serial != run.tuning and run.direction in ("bidir", "chunk_causal") else shared
    own, own_mt, fl, alg_out = flops_of(run, B, H, dk, dv, T, ndir)
    for k, v in fl.items():
        if k in kern:
            kern[k]["executed_tflops"] = v / kern[k]["launches_per_step"] / (kern[k]["avg_ms"] / 1e3) / 1e12
    hbm_step, hbm_src = 0.0, {}
    for k in kern:
        by = read_traffic(k, tag)
        if by is None:
            hbm_step = None
            break
        kern[k]["hbm_gbs"] = by / (kern[k]["avg_ms"] / 1e3) / 1e9
        hbm_step += by * kern[k]["launches_per_step"]
    res = {
        "workload": w.name, "direction": "stream" if run.stream_mode else run.direction,
        "ms_per_step": ms, "tokens_per_s": B * T / (ms / 1e3),
        "segment_tokens": run.L or None,
        "own_gflop": own / 1e9, "own_tflops": own / (ms / 1e3) / 1e12,
        "pct_peak": 100 * own / (ms / 1e3) / 1e12 / peak_tflops,
        "own_with_map_term_gflop": own_mt / 1e9,
        "pct_peak_with_map_term": 100 * own_mt / (ms / 1e3) / 1e12 / peak_tflops,
        "executed_gflop": sum(fl.values()) / 1e9,
        "canonical_frame_gflop": canonical_flops(w.tokens_per_frame, dk, dv) * B * H * w.frames * ndir / 1e9,
        "recurrent_min_gflop": 6 * dk * dv * B * H * T * ndir / 1e9,
        "algorithmic_bytes": algorithmic_bytes(B, T, H, dk, dv),
        "hbm": None if hbm_step is None else {
            "bytes_per_step": hbm_step, "gbs": hbm_step / (ms / 1e3) / 1e9, "peak_gbs": PEAK_HBM_GBS,
            "frac": hbm_step / (ms / 1e3) / 1e9 / PEAK_HBM_GBS,
            "source": f"profiles/<kernel>_{tag}_counters.json (rocprofv3 FETCH_SIZE, WRITE_SIZE)"},
        "kernels": kern,
        "kernels_in_schedule": shared if shared is not kern else None,
    }
    return res, alg_out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="clip60s_121x880_h20d112")
    ap.add_argument("--direction", default=None, choices=["fwd", "bwd", "bidir", "chunk_causal"])
    ap.add_argument("--chunks", default="4,3",
                    help="chunk_causal: frames of the first chunk and of every later chunk")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--segment", type=int, default=0, help="tokens per segment (0 = automatic)")
    ap.add_argument("--serial-scans", action="store_true",
                    help="run a two-scan call's kernels in order on one stream")
    ap.add_argument("--intra", default="sequential", choices=["sequential", "jacobi"],
                    help="transition inside a frame: token-wise (the layer) or the frame-level form; "
                         "jacobi runs with the spatial key scale 1/sqrt(tokens per frame)")
    ap.add_argument("--prologue", default="none", choices=["none", "features"],
                    help="features: raw (unnormalised) q/k through the fused key-feature and query "
                         "normalisation prologue, with the spatial key scale 1/sqrt(d_k * tokens per frame)")
    ap.add_argument("--inverse-reuse", default="on", choices=["on", "off"],
                    help="on: the output kernel of a forward- or backward-only call loads the "
                         "segment-map kernel's sub-chunk inverses (identical results); off: it forms them again")
    ap.add_argument("--no-strip-scan", action="store_true",
                    help="short single-scan calls (one streaming frame) through segment maps and chain")
    ap.add_argument("--parity-procs", type=int, default=16,
                    help="processes of the all-cores oracle run (capped by the host's CPUs)")
    ap.add_argument("--no-parity", action="store_true", help="skip the oracle check and CPU baseline")
    ap.add_argument("--no-extras", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after timing, run one device-to-device copy of this many bytes (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        sys.exit(f"bench.py measures one GPU only (got --gpus {args.gpus}); the layer's multi-GPU "
                 "sharding is described in the design notes and not implemented")

    import torch
    import gated_delta_rule_frame_amd as G
    from gdn_inputs import WORKLOADS

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    cus, mhz, peak_tflops, peak_src = device_peak()
    byname = {wl.name: wl for wl in WORKLOADS}
    w = byname[args.workload]
    pro = args.prologue == "features"
    if pro:
        w = w.resized(qk_spread=1.0)
    stream = w.mode == "step"
    direction = "stream" if stream else (args.direction or "bidir")
    chunks = tuple(int(c) for c in args.chunks.split(","))
    tun = G.Tuning(segment_tokens=args.segment, serial_scans=args.serial_scans,
                   form_inverse=args.inverse_reuse == "off", no_strip_scan=args.no_strip_scan)
    jac = args.intra == "jacobi"
    cc = direction == "chunk_causal"
    # name of the committed counter summaries for this configuration
    tag = w.name + ("_" + direction if direction in ("fwd", "bwd") else "") + ("_jacobi" if jac else "") + \
        ("_features" if pro else "") + ("_chunk_causal" if cc else "") + \
        ("" if args.inverse_reuse == "on" or jac or direction in ("bidir", "chunk_causal", "stream")
         else "_inverse_formed") + ("_no_strip_scan" if args.no_strip_scan else "")
    print(f"[bench] {w.name} {direction}: generating inputs", file=sys.stderr, flush=True)
    run = Run(G, torch, w, direction, args.seed, args.intra, args.prologue, chunks, tun)
    B, T, H, dk, dv = w.batch, w.tokens, w.heads, w.d_k, w.d_v
    key_scale = run.key_scale

    # ---- parity on sampled heads + CPU baselines (the same oracle runs)
    run.step()
    torch.cuda.synchronize()
    parity, cpu_baseline = None, None
    if not args.no_parity:
        pairs_all = [(b, h) for b in range(B) for h in range(H)]
        procs = max(1, min(args.parity_procs, os.cpu_count() or 1, len(pairs_all)))
        # all-cores run: as many heads as one round of the pool covers (every head of the clips)
        pool_pairs = pairs_all if len(pairs_all) <= 2 * procs else pairs_all[:procs]
        print(f"[bench] oracle on {len(pool_pairs)} heads in {procs} processes", file=sys.stderr, flush=True)
        res, wall, _ = oracle_pool(run.x, pool_pairs, run.kind(), run.key_scale, w.tokens_per_frame, chunks, procs)
        one_pair = [pool_pairs[min(7, len(pool_pairs) - 1)]]
        print("[bench] oracle on one head, one thread", file=sys.stderr, flush=True)
        res1, secs1 = run.oracle_local(one_pair)
        res.update(res1)
        parity = run.parity(pool_pairs, res)
        if not parity["pass"]:
            print(json.dumps({"metric": METRIC, "error": "parity failed", "parity": parity}))
            sys.exit(1)
        heads_total = B * H
        cpu_baseline = {
            "value": B * T * len(pool_pairs) / wall / heads_total, "unit": "tokens/s", "cores": procs,
            "kind": "oracle",
            "sample": f"float64 NumPy oracle, {run.kind()[0]} over all {T} tokens of {len(pool_pairs)} of "
                      f"{heads_total} (batch, head) pairs in {procs} processes of one thread each "
                      f"({wall:.1f} s wall on {cpu_model()}), scaled to {heads_total} pairs",
            "single_core": {"value": B * T / secs1 / heads_total, "unit": "tokens/s", "cores": 1,
                            "sample": f"one pair on one thread ({secs1:.1f} s), scaled to {heads_total} pairs"},
        }

    # ---- timing
    main_res, alg_out = measure(G, torch, run, args.steps, args.warmup, peak_tflops, tag)
    ms = main_res["ms_per_step"]
    if stream:
        main_res["stream"] = stream_detail(torch, run, max(3, args.steps // 4))
    kern = main_res["kernels"]
    roof = None
    if kern:
        if jac:
            by = jacobi_bytes(w.tokens_per_frame, w.frames, dk, B * H, 2 if direction == "bidir" else 1)
            dom = max(kern, key=lambda k: kern[k]["avg_ms"] * kern[k]["launches_per_step"])
            achieved = by.get(dom, 0) / kern[dom]["launches_per_step"] / (kern[dom]["avg_ms"] / 1e3) / 1e9
            roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": achieved / PEAK_HBM_GBS, "traffic": read_traffic(dom, tag), "kernel": dom,
                    "bytes_per_launch": by.get(dom, 0) / kern[dom]["launches_per_step"], "avg_ms": kern[dom]["avg_ms"]}
        elif "seg_out_kernel" in kern and alg_out:
            k = kern["seg_out_kernel"]
            # credited flops of one launch: a launch covers one scan direction of
            # the sequence (the mean of the two launches of a chunk-causal call;
            # one call's frame in the streaming loop)
            per_launch = alg_out
            achieved = per_launch / (k["avg_ms"] / 1e3) / 1e12
            roof = {"bound": "mfma", "achieved": achieved, "peak": peak_tflops, "unit": "TFLOP/s",
                    "frac": achieved / peak_tflops, "traffic": read_traffic("seg_out_kernel", tag),
                    "kernel": "seg_out_kernel", "flop_per_launch": per_launch, "avg_ms": k["avg_ms"]}
    if "prologue_kernel" in kern:
        esz = 2 if w.qkv_dtype == "bf16" else 4
        pb = B * T * H * (2 * dk * esz + 8)
        kern["prologue_kernel"]["gbs"] = pb / kern["prologue_kernel"]["launches_per_step"] / \
            (kern["prologue_kernel"]["avg_ms"] / 1e3) / 1e9

    if args.copy_bytes > 0:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE under rocprofv3
        # calibrate the byte counters read for the layer's kernels
        src = torch.empty(args.copy_bytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- secondary workloads (default run only)
    extras = []
    default_main = args.workload == "clip60s_121x880_h20d112" and direction == "bidir" and not (jac or pro) \
        and args.segment == 0 and not args.serial_scans
    if default_main and not args.no_extras:
        del run
        torch.cuda.empty_cache()
        cases = [("clip60s_121x880_h20d112", "fwd"), ("clip5s_21x880_h20d112", "bidir"),
                 ("batched_b2_121x880_h35d64", "bidir"), ("batched_b2_121x880_h35d64", "fwd"),
                 ("stream60s_121x880_h20d112", "stream")]
        for name, dr in cases:
            we = byname[name]
            print(f"[bench] secondary: {name} {dr}", file=sys.stderr, flush=True)
            r = Run(G, torch, we, dr, args.seed)
            r.step()
            torch.cuda.synchronize()
            pe = None
            if not args.no_parity:
                pair = (we.batch - 1, we.heads - 1)
                res1, _ = r.oracle_local([pair])
                pe = r.parity([pair], res1)
            etag = we.name + ("_fwd" if dr == "fwd" else "")
            m, _ = measure(G, torch, r, args.steps, min(args.warmup, 5), peak_tflops, etag)
            if dr == "stream":
                m["stream"] = stream_detail(torch, r, max(3, args.steps // 4))
            m["parity"] = pe
            extras.append(m)
            del r
            torch.cuda.empty_cache()

    line = {
        "metric": METRIC,
        "value": B * T / (ms / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": w.name, "direction": direction, "batch": B, "heads": H, "d_k": dk, "d_v": dv,
            "frames": w.frames, "tokens_per_frame": w.tokens_per_frame, "tokens": T,
            "inputs": f"{w.qkv_dtype} q/k/v, fp32 log-gate/beta/state, fp32 out; fp16 MFMA operands, fp32 accumulation",
            "segment_tokens": main_res["segment_tokens"], "seed": args.seed,
            "intra": args.intra, "key_scale": key_scale, "prologue": args.prologue,
            "chunks_frames": list(chunks) if cc else None, "serial_scans": args.serial_scans,
            "inverse_reuse": None if jac or direction in ("bidir", "chunk_causal") else args.inverse_reuse == "on",
        },
        "peak": {"tflops": peak_tflops, "compute_units": cus, "sclk_mhz": mhz, "flop_per_clk_cu": FLOP_PER_CLK_CU,
                 "source": peak_src, "hbm_gbs": PEAK_HBM_GBS},
        "layer": {k: main_res[k] for k in ("own_gflop", "own_tflops", "pct_peak", "own_with_map_term_gflop",
                                           "pct_peak_with_map_term", "executed_gflop", "canonical_frame_gflop",
                                           "recurrent_min_gflop", "algorithmic_bytes", "hbm")},
        "kernels": kern,
        "parity": parity,
        "roofline": roof,
        "cpu_baseline": cpu_baseline,
        "stream": main_res.get("stream"),
        "secondary": extras or None,
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
