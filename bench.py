#!/usr/bin/env python3
"""One-GPU benchmark of the frame-wise gated delta rule layer forward.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one whole-sequence layer forward (gdn_forward) over one batch of
synthetic inputs already resident in HBM.  The default workload is the 60 s
720p clip: batch 1, 20 heads x 112, 121 latent frames x 880 tokens (106,480
tokens), bf16 q/k/v, fp32 gates/state/accumulation and fp32 output, run in
bidirectional mode (forward scan + reversed scan, summed), as in the SANA-WM
summary page, section 3.2 "Bidirectional and Chunk-Causal GDN Variants".

Before timing, the run checks parity against the float64 CPU oracle on one
sampled head over the whole sequence (heads are independent, so that head's
outputs and final state are exact targets); that same oracle run, limited to
one CPU thread, is the reported CPU baseline.  Prints exactly one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN layer fwd tokens/s & % bf16 MFMA peak, 121×880-token 60 s clip, 1 GPU"
PEAK_TFLOPS = 2516.6        # MI355X dense fp16/bf16 MFMA, 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
TOL = {"f32": 1e-4, "bf16": 2e-2}
KERNEL_SOURCES = ("gdn_chunked.hip", "gdn_prologue.hip", "gdn_mfma.h", "gdn_common.h")


# --------------------------------------------------------------- FLOP models

def canonical_flops(C, dk, dv):
    """Frame-as-chunk count per (batch, head, frame, direction): strict-lower
    K K^T plus forward substitution on [W|U], causal Q K^T and its product with
    U', and the three C x d x d state products."""
    return C * (C - 1) * (2 * dk + dv) + C * (C + 1) * (dk + dv) + 6 * C * dk * dv


def subchunk_sizes(T, L, c=64):
    """Token counts of the 64-token sub-chunks, per segment of L tokens."""
    segs = []
    for s0 in range(0, T, L):
        n = min(L, T - s0)
        segs.append([min(c, n - a) for a in range(0, n, c)])
    return segs


def out_flops(n, d, inverse=True):
    """Algorithmic flops of the output pass on one sub-chunk of n tokens:
    causal Q K^T, K H and Q H, Tm diag(beta) R and P V' (triangular), the
    state update, and (inverse: unless it loads the map kernel's) the
    strict-lower K K^T and the triangular inverse (n^3/3)."""
    tri = n * (n - 1) * d + n ** 3 // 3 if inverse else 0
    return tri + 3 * n * (n + 1) * d + 6 * n * d * d


def map_flops(n, d, q_only=False):
    """Algorithmic flops of the segment-map pass on one sub-chunk (state [P|Q],
    2d columns; q_only: Q alone, d columns): strict-lower K K^T, the inverse,
    K X, Tm diag(beta) R and the state update."""
    w = 1 if q_only else 2
    return n * (n - 1) * d + w * n * (n + 1) * d + 4 * w * n * d * d + n ** 3 // 3


def executed_flops(T, L, d, bh, ndir, reuse=True):
    """Algorithmic flops per call of each of the chunked path's kernels, summed
    over its launches (a bidirectional call launches each kernel once per scan
    direction).  reuse: the output kernel of a forward- or backward-only call
    loads the map kernel's sub-chunk inverses (the library default; with more
    than one segment), and the map kernel then covers every segment."""
    segs = subchunk_sizes(T, L)
    reuse = reuse and len(segs) > 1 and ndir == 1
    per_out = sum(out_flops(n, d, inverse=not reuse) for seg in segs for n in seg)
    if ndir == 1:
        # maps of every segment but the last of the scan (all with reuse)
        maps = sum(map_flops(n, d) for seg in (segs if reuse else segs[:-1]) for n in seg)
    else:
        # forward maps of every segment (the last one's P, transposed, is the
        # reversed scan's first), reversed maps (Q only) of all but the first
        maps = sum(map_flops(n, d) for seg in segs for n in seg)
        maps += sum(map_flops(n, d, q_only=True) for seg in segs[1:] for n in seg)
    chain = (len(segs) - 1) * 2 * d ** 3
    return {"seg_out_kernel": per_out * bh * ndir, "seg_map_kernel": maps * bh,
            "seg_chain_kernel": chain * bh * ndir}


def chunk_causal_flops(T, S, L, d, bh, first, every):
    """Per-call flops of the chunk-causal layer on the chunked path: the
    forward scan's maps, chain and outputs, and the reversed scan's outputs
    over each chunk of frames (its segments are the chunks: no maps, no
    chain, so they always form their inverses)."""
    fl = executed_flops(T, L, d, bh, 1, reuse=False)   # two-scan calls form their inverses
    bounds, t0, n = [], 0, first * S
    while t0 < T:
        bounds.append((t0, min(T, t0 + n)))
        t0, n = t0 + n, every * S
    rev = sum(out_flops(min(64, e - a), d) for s0, s1 in bounds for a in range(s0, s1, 64) for e in [s1])
    fl["seg_out_kernel"] += rev * bh
    return fl


def jacobi_flops(S, F, d, bh, ndir):
    """Algorithmic flops per call of the frame-level (Jacobi) path, per kernel:
    per frame c^2 K^T diag(beta) K and c K^T diag(beta) V (4 S d^2), the
    outputs Q H_end (2 S d^2, one product with the summed state), and one
    d x d state product per frame and scan in the chain (2 d^3)."""
    return {"jac_map_kernel": 4 * S * d * d * F * bh, "jac_out_kernel": 2 * S * d * d * F * bh,
            "seg_chain_kernel": 2 * d ** 3 * F * bh * ndir}


def jacobi_bytes(S, F, d, bh, ndir, out_bytes=4):
    """Algorithmic HBM bytes per call of the frame-level path, per kernel: the
    map kernel reads K, V (bf16) and beta and writes one [P | Q] map per frame
    and scan (fp32); the output kernel reads Q and the end states and writes
    the outputs; the chain reads the maps and writes the states."""
    T = S * F
    maps = ndir * F * bh * d * 2 * d * 4
    states = ndir * (F + 1) * bh * d * d * 4
    return {"jac_map_kernel": T * bh * (2 * d * 2 + 4) + maps,
            "jac_out_kernel": T * bh * (2 * d + out_bytes * d) + states,
            "seg_chain_kernel": maps + states}


def kernel_source_hash():
    """Hash of the kernel sources without their // comments and with runs of
    whitespace collapsed: a change of wording alone keeps the counters valid."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "gated_delta_rule_frame_amd", "csrc", f)) as fh:
            code = re.sub(r"//[^\n]*", "", fh.read())
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def read_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if it is missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.json")
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


# --------------------------------------------------------------------- main

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
    ap.add_argument("--parity-head", type=int, default=7)
    ap.add_argument("--parity-heads", type=int, default=3,
                    help="heads checked against the oracle (the parity head, then the first and the last)")
    ap.add_argument("--intra", default="sequential", choices=["sequential", "jacobi"],
                    help="transition inside a frame: token-wise (the layer) or the frame-level form; "
                         "jacobi runs with the spatial key scale 1/sqrt(tokens per frame)")
    ap.add_argument("--prologue", default="none", choices=["none", "features"],
                    help="features: raw (unnormalised) q/k through the fused key-feature and query "
                         "normalisation prologue, with the spatial key scale 1/sqrt(d_k * tokens per frame)")
    ap.add_argument("--inverse-reuse", default="on", choices=["on", "off"],
                    help="on: the output kernel of a forward- or backward-only call loads the "
                         "segment-map kernel's sub-chunk inverses (identical results); off: it forms them again")
    ap.add_argument("--no-parity", action="store_true", help="skip the oracle check and CPU baseline")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after timing, run one device-to-device copy of this many bytes (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        sys.exit(f"bench.py measures one GPU only (got --gpus {args.gpus}); the layer's multi-GPU "
                 "sharding is described in the design notes and not implemented")

    import torch
    import gated_delta_rule_frame_amd as G
    from gdn_inputs import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    w = {wl.name: wl for wl in WORKLOADS}[args.workload]
    pro = args.prologue == "features"
    if pro:
        w = w.resized(qk_spread=1.0)
    direction = args.direction or ("bidir" if w.mode == "bidir" else "fwd")
    dev = torch.device("cuda:0")
    G.set_segment_tokens(args.segment)
    G.set_inverse_reuse(args.inverse_reuse == "on")

    x = make_inputs(w, args.seed)
    qkv_dt = torch.bfloat16 if w.qkv_dtype == "bf16" else torch.float32
    d = {n: torch.from_numpy(x[n]).to(dev, qkv_dt) for n in ("q", "k", "v")}
    for n in ("log_gate", "beta"):
        d[n] = torch.from_numpy(x[n]).to(dev)
    h0 = torch.from_numpy(x["h0"]).to(dev) if np.any(x["h0"]) else None
    B, T, H, dk, dv = w.batch, w.tokens, w.heads, w.d_k, w.d_v
    jac = args.intra == "jacobi"
    key_scale = (dk * w.tokens_per_frame) ** -0.5 if pro else w.tokens_per_frame ** -0.5 if jac else 1.0
    first_cf, every_cf = (int(c) for c in args.chunks.split(","))
    cc = direction == "chunk_causal"
    # name of the committed counter summaries for this configuration
    tag = w.name + ("_" + direction if direction in ("fwd", "bwd") else "") + ("_jacobi" if jac else "") + \
        ("_features" if pro else "") + ("_chunk_causal" if cc else "") + \
        ("" if args.inverse_reuse == "on" or jac or direction in ("bidir", "chunk_causal") else "_inverse_formed")
    prob = G.make_problem(B, H, dk, dv, w.frames, w.tokens_per_frame, G.BF16 if w.qkv_dtype == "bf16" else G.F32,
                          G.F32, "auto", key_scale, args.intra, first_cf, every_cf, args.prologue)
    ws = torch.empty(max(G.workspace_size(prob, direction), 16), dtype=torch.uint8, device=dev)
    out = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    hT = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)

    def step():
        G.forward(d["q"], d["k"], d["v"], d["log_gate"], d["beta"], h0, direction,
                  tokens_per_frame=w.tokens_per_frame, out=out, final_state=hT, workspace=ws,
                  key_scale=key_scale, intra=args.intra, first_chunk_frames=first_cf, chunk_frames=every_cf,
                  prologue=args.prologue)

    # ---- parity on sampled heads + CPU baseline (the same oracle runs)
    parity, cpu_baseline = None, None
    step()
    torch.cuda.synchronize()
    if not args.no_parity:
        from threadpoolctl import threadpool_limits
        from oracle import gdn_oracle as O
        # the requested head, then the first and the last (of batch 0): about
        # 10 s of single-thread oracle work at the 60 s clip
        heads = []
        for hh in (min(args.parity_head, H - 1), 0, H - 1)[:max(1, args.parity_heads)]:
            if hh not in heads:
                heads.append(hh)
        rel = lambda u, r: float(np.max(np.abs(u - r)) / np.sqrt(np.mean(r * r)))
        tol = TOL[w.qkv_dtype]
        cpu_s, errs = 0.0, []
        for hh in heads:
            a = [x[n][:1, :, hh:hh + 1] for n in ("q", "k", "v", "log_gate", "beta")]
            with threadpool_limits(1):
                t0 = time.perf_counter()
                if pro:
                    a[0], a[1] = O.query_features(a[0]), O.key_features(a[1])
                if jac:
                    ro, rH = O.jacobi_forward(direction, *a, x["h0"][:1, hh:hh + 1], key_scale=key_scale,
                                              tokens_per_frame=w.tokens_per_frame)
                elif cc:
                    ro, rH = O.chunk_causal(*a, x["h0"][:1, hh:hh + 1], key_scale=key_scale,
                                            tokens_per_frame=w.tokens_per_frame,
                                            first_chunk_frames=first_cf, chunk_frames=every_cf)
                else:
                    ro, rH = O.forward(direction, *a, x["h0"][:1, hh:hh + 1], key_scale=key_scale)
                cpu_s += time.perf_counter() - t0
            o = out[:1, :, hh:hh + 1].double().cpu().numpy()
            s_ = hT[:1, hh:hh + 1].double().cpu().numpy()
            errs.append((hh, rel(o, ro), rel(s_, rH)))
        eo, es = max(e[1] for e in errs), max(e[2] for e in errs)
        parity = {"heads": heads, "out_err": eo, "state_err": es, "tol": tol, "pass": eo <= tol and es <= tol,
                  "per_head": {str(hh): [round(a_, 6), round(b_, 6)] for hh, a_, b_ in errs}}
        if not parity["pass"]:
            print(json.dumps({"metric": METRIC, "error": "parity failed", "parity": parity}))
            sys.exit(1)
        # oracle tokens/s for the whole workload: it handled len(heads) of B*H heads
        cpu_rate = T * len(heads) / cpu_s / (B * H)
        cpu_baseline = {"value": cpu_rate, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                        "sample": f"float64 NumPy oracle, {direction} over all {T} tokens of {len(heads)} of "
                                  f"{B * H} heads ({cpu_s:.1f} s on 1 thread of {cpu_model()}), scaled to "
                                  f"{B * H} heads"}

    # ---- timing
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    G.profile_reset()
    G.profile_enable(True)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    G.profile_enable(False)
    ms = ev0.elapsed_time(ev1) / args.steps
    prof = G.profile_read()

    if args.copy_bytes > 0:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE under rocprofv3
        # calibrate the byte counters read for the layer's kernels
        src = torch.empty(args.copy_bytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    tokens_per_s = B * T / (ms / 1e3)
    ndir = 2 if direction in ("bidir", "chunk_causal") else 1
    L = G.segment_plan(prob, direction) if hasattr(G, "segment_plan") else None
    canon = canonical_flops(w.tokens_per_frame, dk, dv) * B * H * w.frames * ndir
    kern = {k: {"launches": n, "avg_ms": (t / n if n else None)} for k, (n, t) in prof.items() if n}
    roof, flops_exec = None, None
    if jac and kern:
        F_, S_ = w.frames, w.tokens_per_frame
        fl = jacobi_flops(S_, F_, dk, B * H, ndir)
        by = jacobi_bytes(S_, F_, dk, B * H, ndir)
        flops_exec = sum(fl.values())
        for k in fl:
            if k in kern:
                launches = kern[k]["launches"] / args.steps
                kern[k]["tflops"] = fl[k] / launches / (kern[k]["avg_ms"] / 1e3) / 1e12
                kern[k]["gbs"] = by[k] / launches / (kern[k]["avg_ms"] / 1e3) / 1e9
        dom = max(kern, key=lambda k: kern[k]["avg_ms"] * kern[k]["launches"])
        achieved = kern[dom].get("gbs", 0.0)
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": read_traffic(dom, tag), "kernel": dom}
    elif "seg_out_kernel" in kern and L:
        reuse = args.inverse_reuse == "on"
        fl = (chunk_causal_flops(T, w.tokens_per_frame, L, dk, B * H, first_cf, every_cf) if cc
              else executed_flops(T, L, dk, B * H, ndir, reuse))
        flops_exec = sum(fl.values())   # per call
        per_launch = {}
        for k in fl:
            if k in kern:
                # launches of k per call, from the profile of the timed steps
                per_launch[k] = fl[k] * args.steps / kern[k]["launches"]
                kern[k]["tflops"] = per_launch[k] / (kern[k]["avg_ms"] / 1e3) / 1e12
        dom = max(kern, key=lambda k: kern[k]["avg_ms"] * kern[k]["launches"])
        achieved = per_launch.get(dom, 0) / (kern[dom]["avg_ms"] / 1e3) / 1e12
        traffic = read_traffic(dom, tag)
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_TFLOPS, "traffic": traffic, "kernel": dom}
    if "prologue_kernel" in kern:
        # algorithmic bytes: q and k read once, two fp32 factors per (token, head) written
        esz = 2 if w.qkv_dtype == "bf16" else 4
        pb = B * T * H * (2 * dk * esz + 8)
        launches = kern["prologue_kernel"]["launches"] / args.steps
        kern["prologue_kernel"]["gbs"] = pb / launches / (kern["prologue_kernel"]["avg_ms"] / 1e3) / 1e9
    credited = flops_exec if jac else (min(canon, flops_exec) if flops_exec else canon)
    layer_tflops = credited / (ms / 1e3) / 1e12

    line = {
        "metric": METRIC,
        "value": tokens_per_s,
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
            "segment_tokens": None if jac else L, "seed": args.seed,
            "intra": args.intra, "key_scale": key_scale, "prologue": args.prologue,
            "chunks_frames": [first_cf, every_cf] if cc else None,
            "inverse_reuse": None if jac or direction in ("bidir", "chunk_causal") else args.inverse_reuse == "on",
        },
        "layer": {"canonical_gflop": canon / 1e9, "executed_gflop": (flops_exec or 0) / 1e9,
                  "credited_tflops": layer_tflops, "pct_peak": 100 * layer_tflops / PEAK_TFLOPS,
                  "recurrent_min_gflop": 6 * dk * dv * B * H * T * ndir / 1e9},
        "kernels": kern,
        "parity": parity,
        "roofline": roof,
        "cpu_baseline": cpu_baseline,
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
