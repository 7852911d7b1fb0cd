#!/usr/bin/env python3
"""Benchmark of one Video DeltaNet hybrid video-to-video attention layer
forward on one MI355X, at the 768p shape (B=1, H=24, d=128, 60 latent frames x
1008 tokens = 60,480 video tokens, 512 text tokens, bf16).

A step is one call of the whole layer (vdn_hybrid_attn_fwd: the VDA branch -
statistics, factor and V^T copy in one pass, then the bidirectional scan -
followed by the block-sparse softmax with the merge fused into its epilogue)
on synthetic inputs already resident in HBM.  Prints one JSON line: layer
throughput in video tokens/s (warm; cold runs with the caches flushed are
reported beside it), the roofline of the dominant kernel (the fused softmax +
merge, launched alone as the layer's second stage and timed with HIP events
on its stream), the VDA branch against the HBM roof, the same layer on the
long (120-frame) and the stress (batch 2, ill-conditioned) shapes, an fp32
layer on the fp32 matrix cores (4 heads, 20 frames of the 768p frame), and the
CPU oracle timed on a bounded sample of the 768p workload.  It also times the
layer followed by the two branches' separate output projections (d_model =
H*d), the projection product alone and the library matmul on the same
operands, and the backward pass.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0
PEAK_FP32_TFLOPS = 157.3      # MI355X dense fp32 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k1_softmax_768p_hbm_traffic.md")
VDA_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "vda_branch_768p_hbm_traffic.md")
VDA_SOURCES = ["video_diffusion_hybrid_block_amd/csrc/k_vda_stats.hip",
               "video_diffusion_hybrid_block_amd/csrc/k_scan.hip",
               "video_diffusion_hybrid_block_amd/csrc/vdn_device.h",
               "video_diffusion_hybrid_block_amd/csrc/vdn_internal.h"]
K1_SOURCES = ["video_diffusion_hybrid_block_amd/csrc/k_softmax.hip",
              "video_diffusion_hybrid_block_amd/csrc/vdn_device.h",
              "video_diffusion_hybrid_block_amd/csrc/vdn_internal.h"]


def visible_keys_per_frame(w):
    """Keys one query of frame t scores: video tokens of the visible frames
    (own chunk +- window, plus the first/last frame; anchors see everything)
    and all text tokens."""
    T, C, wc = w.frames, w.chunk_frames, w.window_chunks
    out = []
    for t in range(T):
        if t in (0, T - 1):
            nf = T
        else:
            c = t // C
            lo, hi = max(0, (c - wc) * C), min(T, (c + wc + 1) * C) - 1
            vis = set(range(lo, hi + 1)) | {0, T - 1}
            nf = len(vis)
        out.append(nf * w.tokens_per_frame + w.text_tokens)
    return out


def softmax_flops(w):
    """Algorithmic work of the fused softmax + merge stage: 4*d flops (q.k and
    p*v) per visible (query, key) pair plus 2*d*d for the linear read R q of
    every video query, all batches and heads."""
    pairs = sum(k * w.tokens_per_frame for k in visible_keys_per_frame(w))
    read = 2.0 * w.head_dim * w.head_dim * w.video_tokens
    return (4.0 * w.head_dim * pairs + read) * w.batch * w.heads


def sources_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(path=TRAFFIC_FILE, sources=K1_SOURCES, key="traffic_bytes_per_launch"):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].split(": ", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("sources_sha256_16") != sources_hash(sources):
        return None
    try:
        return int(float(vals[key]))
    except (KeyError, ValueError):
        return None


def scan_frames(w):
    """Frames the forward and the backward state fold (non-anchor frames
    before the window of the last chunk that has a non-anchor frame, resp.
    after the window of the first one)."""
    T, C, wc = w.frames, w.chunk_frames, w.window_chunks
    nc = -(-T // C)
    anchors = {0, T - 1}
    win_lo = lambda c: max(0, (c - wc) * C)
    win_hi = lambda c: min(T, (c + wc + 1) * C) - 1
    has_query = lambda c: any(t not in anchors for t in range(c * C, min((c + 1) * C, T)))
    fend = next((win_lo(c) for c in reversed(range(nc)) if has_query(c)), 0)
    fbeg = next((win_hi(c) for c in range(nc) if has_query(c)), T - 1)
    fwd = [f for f in range(T) if f < fend and f not in anchors]
    bwd = [f for f in range(T) if f > fbeg and f not in anchors]
    return fwd, bwd, nc


def vda_bytes(w):
    """Bytes the VDA branch must move as built, all batches and heads, each
    counted once: K, V and beta of the frames it folds (V of every frame and
    the text, for the V^T copy), the V^T copy written, G (bf16 hi + lo) and B
    written by the statistics pass and read once per fold step by the scan,
    the chunk snapshots written, and the combine's reads and writes."""
    fwd, bwd, nc = scan_frames(w)
    stat = len(set(fwd) | set(bwd))
    P, L, T, d = w.tokens_per_frame, w.text_tokens, w.frames, w.head_dim
    mat = d * d * 4
    stats = (T * P + L) * d * 2 + (stat * P + L) * d * 2 + (stat * P + L) * 4 \
        + (T * P + L) * d * 2 + (stat + 1) * 2 * mat
    text_step = 1 if L else 0
    scan = (len(fwd) + len(bwd) + 2 * text_step) * 2 * mat + 2 * (nc + 1) * mat
    combine = 3 * (nc + 1) * mat
    return (stats + scan + combine) * w.batch * w.heads


def cpu_info():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model


def cpu_baseline(w, inp, budget_s=20.0):
    """The float64 oracle on a bounded sample of whole heads: heads of batch 0
    in turn, each its complete forward (every video token: the softmax of
    every frame, the frame statistics and every frame's state folds), until
    about budget_s seconds of CPU work; the layer's time is the mean head's
    time x B x H (heads are independent and of equal size)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import vdn_oracle as O
    from video_diffusion_hybrid_block_amd import synth
    lay = O.Layout(**synth.layout_kwargs(w))
    tokens = np.arange(w.video_tokens)
    t_start = time.perf_counter()
    per_head = []
    while len(per_head) < w.heads and (not per_head or time.perf_counter() - t_start < budget_s):
        t0 = time.perf_counter()
        O.hybrid_attn_rows(inp, lay, 0, len(per_head), tokens)
        per_head.append(time.perf_counter() - t0)
    layer_s = sum(per_head) / len(per_head) * w.batch * w.heads
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": w.batch * w.video_tokens / layer_s, "unit": "video tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{len(per_head)} of {w.batch * w.heads} (batch, head) pairs, each the "
                      f"oracle's complete forward of one head ({w.video_tokens} queries), "
                      f"{sum(per_head):.1f} s; layer time = mean head x {w.batch * w.heads} = "
                      f"{layer_s:.0f} s",
            "affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": cpu_info()}


def time_calls(fn, steps, warmup, stream, flush=None):
    """Warm: `steps` back-to-back calls between two events (mean) and each
    call between its own events (median, min).  Cold (flush given): each call
    after the flush, its own events around the call only."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    mean = e0.elapsed_time(e1) / steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    each = sorted(a.elapsed_time(b) for a, b in ev)
    out = {"mean": mean, "median": each[len(each) // 2], "min": each[0]}
    if flush is not None:
        cold = []
        for _ in range(steps):
            flush()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            cold.append(a.elapsed_time(b))
        cold.sort()
        out["cold_median"] = cold[len(cold) // 2]
        out["cold_min"] = cold[0]
    return out


def fp32_figures(steps, warmup):
    """An fp32 layer (softmax with the fused merge, statistics and scan on the
    fp32 matrix cores): the whole layer and the softmax alone
    (vdn_softmax_fwd), which carries the layer's flops."""
    import torch

    from video_diffusion_hybrid_block_amd import binding as V
    from video_diffusion_hybrid_block_amd import synth
    w = synth.Workload("fp32_4h_20f", 1, 4, 128, 20, 1008, 512, "f32", 2024, chunk_frames=5,
                       window_chunks=1)
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    inp = synth.make_inputs(w)
    dev = {k: torch.from_numpy(a).float().cuda() for k, a in inp.items()}
    geo = dict(frames=w.frames, tokens_per_frame=w.tokens_per_frame, chunk_frames=w.chunk_frames,
               window_chunks=w.window_chunks)
    out = torch.empty_like(dev["q"])
    o_soft = torch.empty_like(dev["q"])

    def layer():
        V.hybrid_attn(dev["q"], dev["k"], dev["v"], dev["text_k"], dev["text_v"], dev["beta"],
                      dev["alpha"], dev["gate_logits"], **geo, out=out)

    def softmax():
        V.softmax_fwd(dev["q"], dev["k"], dev["v"], dev["text_k"], dev["text_v"], **geo, out=o_soft)

    stream = torch.cuda.current_stream()
    lay_t = time_calls(layer, steps, warmup, stream)
    sm_t = time_calls(softmax, steps, 2, stream)
    fl = softmax_flops(w)
    return {"workload": f"B={w.batch} H={w.heads} d={w.head_dim} T={w.frames} "
                        f"P={w.tokens_per_frame} L={w.text_tokens} fp32",
            "layer_ms": round(lay_t["mean"], 4),
            "video_tokens_per_s": round(w.batch * w.video_tokens / (lay_t["mean"] / 1e3), 1),
            "softmax_ms": round(sm_t["mean"], 4),
            "softmax_tflops": round(fl / (sm_t["mean"] / 1e3) / 1e12, 1),
            "softmax_frac_fp32_peak": round(fl / (sm_t["mean"] / 1e3) / 1e12 / PEAK_FP32_TFLOPS, 4)}


def layer_figures(w, steps, warmup, flush=None, keep=False):
    """The layer on workload w: warm (and cold) call times, and its two
    stages launched alone - the VDA branch (vdn_vda_branch, writing the V^T
    copy) and the fused softmax + merge (vdn_softmax_merge_fwd_vt)."""
    import torch

    from video_diffusion_hybrid_block_amd import binding as V
    from video_diffusion_hybrid_block_amd import synth
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    inp = synth.make_inputs(w)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = {}
    for k, a in inp.items():
        t = torch.from_numpy(a)
        if k in ("q", "k", "v", "text_k", "text_v"):
            t = t.to(tdt)
        dev[k] = t.cuda()
    L = w.text_tokens
    geo = dict(frames=w.frames, tokens_per_frame=w.tokens_per_frame, chunk_frames=w.chunk_frames,
               window_chunks=w.window_chunks)
    lay = V.make_layout(batch=w.batch, heads=w.heads, head_dim=w.head_dim, frames=w.frames,
                        tokens_per_frame=w.tokens_per_frame, text_tokens=L, dtype=w.dtype,
                        chunk_frames=w.chunk_frames, window_chunks=w.window_chunks)
    ws = torch.empty(V.workspace_size(lay), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(dev["q"])
    tk, tv = (dev["text_k"], dev["text_v"]) if L else (None, None)
    R, vt = V.vda_branch(dev["k"], dev["v"], tk, tv, dev["beta"], dev["alpha"], want_vt=True,
                         workspace=ws, **geo)

    def layer():
        V.hybrid_attn(dev["q"], dev["k"], dev["v"], tk, tv, dev["beta"], dev["alpha"],
                      dev["gate_logits"], **geo, out=out, workspace=ws)

    def vda():
        V.vda_branch(dev["k"], dev["v"], tk, tv, dev["beta"], dev["alpha"], out=R, vt_out=vt,
                     workspace=ws, **geo)

    def softmax_stage():
        V.softmax_merge_fwd_vt(dev["q"], dev["k"], tk, vt, R, dev["gate_logits"], **geo, out=out)

    stream = torch.cuda.current_stream()
    print(f"[bench] {w.name}: warmup {warmup}, timing {steps} layer steps", file=sys.stderr,
          flush=True)
    t0 = time.perf_counter()
    lay_t = time_calls(layer, steps, warmup, stream, flush)
    wall = time.perf_counter() - t0
    vda_t = time_calls(vda, steps, 2, stream)
    k1_t = time_calls(softmax_stage, steps, 2, stream)
    res = {"w": w, "layer": lay_t, "vda": vda_t, "k1": k1_t, "wall": wall}
    if keep:
        res.update(inp=inp, dev=dev, lay=lay, geo=geo, R=R, stream=stream, tk=tk, tv=tv)
    else:
        del dev, ws, out, R, vt
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="768p")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-proj", action="store_true",
                    help="skip the layer-with-output-projections timing")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward-pass timing")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the long and stress workloads")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(the layer shards by head; see the design notes). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from video_diffusion_hybrid_block_amd import binding as V
    from video_diffusion_hybrid_block_amd import synth

    w = synth.WORKLOADS[args.workload]
    # cold runs: a 512 MiB write between calls evicts the L2s and the MALL
    flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")

    def flush():
        flush_buf.fill_(1)

    head = layer_figures(w, args.steps, args.warmup, flush=flush, keep=True)
    del flush_buf
    torch.cuda.empty_cache()
    inp, dev, lay, geo, R, stream = (head[k] for k in ("inp", "dev", "lay", "geo", "R", "stream"))
    tk, tv = head["tk"], head["tv"]
    L = w.text_tokens
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ms = head["layer"]["mean"]
    k1_ms = head["k1"]["mean"]
    vda_ms = head["vda"]["mean"]
    sws = torch.empty(max(V.softmax_workspace_size(lay), 1), dtype=torch.uint8, device="cuda")

    # the step after the layer: both gated branches through their own output
    # projections (d_model = H*d), as one product (bf16 layouts only)
    proj = None
    if w.dtype == "bf16" and not args.no_proj:
        H, d = w.heads, w.head_dim
        dm = H * d
        w_o = torch.from_numpy(synth.make_proj_weight(dm, H, d, seed=w.seed + 1)).to(tdt).cuda()
        pws = torch.empty(V.proj_workspace_size(lay), dtype=torch.uint8, device="cuda")
        y = torch.empty((w.batch, w.video_tokens, dm), dtype=tdt, device="cuda")
        x2 = V.softmax_branches_fwd(dev["q"], dev["k"], dev["v"], tk, tv, R, dev["gate_logits"],
                                    **geo, workspace=sws).view(w.batch * w.video_tokens, 2 * H * d)
        y2 = torch.empty((w.batch * w.video_tokens, dm), dtype=tdt, device="cuda")

        def layer_proj():
            V.hybrid_attn_proj(dev["q"], dev["k"], dev["v"], tk, tv, dev["beta"], dev["alpha"],
                               dev["gate_logits"], w_o, **geo, out=y, workspace=pws)

        def product():
            V.out_proj(x2, w_o, out=y2)

        wt = w_o.t().contiguous()

        def library_product():
            torch.matmul(x2, wt, out=y2)

        def timed(fn, n):
            for _ in range(2):
                fn()
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(n):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / n

        # FP8 (MXFP8) form: weights quantized once; the layer's softmax kernel
        # writes the activations (both gated branches) as MXFP8 itself
        wq, wsc = V.mxfp8_quantize(w_o)
        xq, xsc = V.mxfp8_quantize(x2)
        pws8 = torch.empty(V.lib().vdn_hybrid_attn_proj_mxfp8_workspace_size(ctypes.byref(lay)),
                           dtype=torch.uint8, device="cuda")

        def layer_proj8():
            V.hybrid_attn_proj_mxfp8(dev["q"], dev["k"], dev["v"], tk, tv, dev["beta"],
                                     dev["alpha"], dev["gate_logits"], wq, wsc, **geo, out=y,
                                     workspace=pws8)

        def product8():
            V.out_proj_mxfp8(xq, xsc, wq, wsc, out=y2)

        print("[bench] layer with output projections", file=sys.stderr, flush=True)
        lp_ms = timed(layer_proj, args.steps)
        pr_ms = timed(product, args.steps)
        lib_ms = timed(library_product, args.steps)
        lp8_ms = timed(layer_proj8, args.steps)
        pr8_ms = timed(product8, args.steps)
        pflops = 2.0 * w.batch * w.video_tokens * (2 * H * d) * dm
        proj = {"d_model": dm, "layer_with_proj_ms": round(lp_ms, 4),
                "video_tokens_per_s": round(w.batch * w.video_tokens / (lp_ms / 1e3), 1),
                "proj_kernel": "proj_gemm_kernel (bf16, 256x256 tiles)",
                "proj_ms": round(pr_ms, 4),
                "proj_tflops": round(pflops / (pr_ms / 1e3) / 1e12, 1),
                "proj_frac": round(pflops / (pr_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "library_matmul_ms": round(lib_ms, 4),
                "fp8": {"format": "MXFP8 (E4M3 codes, E8M0 scale per 32 along K)",
                        "proj_kernel": "proj_mxfp8_kernel (v_mfma_scale_f32_32x32x64_f8f6f4)",
                        "proj_ms": round(pr8_ms, 4),
                        "proj_tflops": round(pflops / (pr8_ms / 1e3) / 1e12, 1),
                        "proj_frac_fp8_peak": round(pflops / (pr8_ms / 1e3) / 1e12 / PEAK_FP8_TFLOPS, 4),
                        "activations": "quantized in the softmax kernel's epilogue "
                                       "(softmax_vt_kernel<128, 4>)",
                        "layer_with_proj_ms": round(lp8_ms, 4),
                        "video_tokens_per_s": round(w.batch * w.video_tokens / (lp8_ms / 1e3), 1)}}
        del pws, pws8, y, y2, x2, w_o, wt, xq, xsc, wq, wsc

    # backward pass of the layer (gradients of every input given dO), bf16
    # layouts only: the forward recomputation plus the backward kernels
    bwd = None
    if w.dtype == "bf16" and not args.no_bwd:
        g = torch.Generator(device="cuda")
        g.manual_seed(w.seed + 2)
        dO = torch.randn(dev["q"].shape, generator=g, device="cuda").to(tdt)
        bws = torch.empty(V.bwd_workspace_size(lay), dtype=torch.uint8, device="cuda")

        def backward():
            return V.hybrid_attn_bwd(dev["q"], dev["k"], dev["v"], tk, tv, dev["beta"],
                                     dev["alpha"], dev["gate_logits"], dO, **geo, workspace=bws)

        print("[bench] backward pass", file=sys.stderr, flush=True)
        for _ in range(2):
            backward()
        torch.cuda.synchronize()
        nb = max(3, args.steps // 4)
        e0.record(stream)
        for _ in range(nb):
            backward()
        e1.record(stream)
        torch.cuda.synchronize()
        b_ms = e0.elapsed_time(e1) / nb
        pairs = sum(k_ * w.tokens_per_frame for k_ in visible_keys_per_frame(w))
        # attention flops of a backward with recomputation: 4d (forward) +
        # 10d (dP, dS.K, dS^T.Q, P^T.dO and the recomputed S) per visible pair
        aflops = 14.0 * w.head_dim * pairs * w.batch * w.heads
        bwd = {"ms": round(b_ms, 3), "calls": nb,
               "video_tokens_per_s": round(w.batch * w.video_tokens / (b_ms / 1e3), 1),
               "attention_tflops": round(aflops / (b_ms / 1e3) / 1e12, 1),
               "note": "vdn_hybrid_attn_bwd: forward recomputation + gradients of q, k, v, "
                       "text k/v, beta, alpha, gate logits (fp32)"}
        del bws

        # training pair: a forward that keeps its residuals, then the backward
        # from them (no recomputation of the softmax forward)
        saved = torch.empty(V.train_saved_size(lay), dtype=torch.uint8, device="cuda")
        o_t = torch.empty_like(dev["q"])

        def fwd_train():
            V.hybrid_attn_fwd_train(dev["q"], dev["k"], dev["v"], tk, tv, dev["beta"],
                                    dev["alpha"], dev["gate_logits"], **geo, out=o_t,
                                    saved=saved)

        def bwd_saved():
            return V.hybrid_attn_bwd_saved(dev["q"], dev["k"], dev["v"], tk, tv, dev["beta"],
                                           dev["alpha"], dev["gate_logits"], dO, saved, **geo)

        print("[bench] training pair", file=sys.stderr, flush=True)
        for _ in range(2):
            fwd_train()
            bwd_saved()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(nb):
            fwd_train()
            bwd_saved()
        e1.record(stream)
        torch.cuda.synchronize()
        t_ms = e0.elapsed_time(e1) / nb
        e0.record(stream)
        for _ in range(nb):
            fwd_train()
        e1.record(stream)
        torch.cuda.synchronize()
        ft_ms = e0.elapsed_time(e1) / nb
        bwd["training_pair"] = {
            "ms": round(t_ms, 3), "fwd_train_ms": round(ft_ms, 3),
            "bwd_saved_ms": round(t_ms - ft_ms, 3),
            "video_tokens_per_s": round(w.batch * w.video_tokens / (t_ms / 1e3), 1),
            "attention_tflops": round(aflops / (t_ms / 1e3) / 1e12, 1),
            "note": "vdn_hybrid_attn_fwd_train + vdn_hybrid_attn_bwd_saved: forward (the layer "
                    "output to rounding, exact fp32 scores) keeping O_soft, RMSNorm(R q), lse, 1/r and the scan states; "
                    "backward from them; 14d flops per visible pair over the pair"}
        del saved, o_t, dO

    if args.copy_calib:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    # the long and the stress workloads: the same figures, fewer steps
    extra = {}
    if not args.no_extra and args.workload == "768p":
        del dev, R, sws
        head.pop("dev")
        head.pop("R")
        torch.cuda.empty_cache()
        for name in ("long_120f", "stress_lowrank"):
            xw = synth.WORKLOADS[name]
            f = layer_figures(xw, max(5, args.steps // 4), 2)
            xfl = softmax_flops(xw)
            extra[name] = {
                "workload": f"B={xw.batch} H={xw.heads} d={xw.head_dim} T={xw.frames} "
                            f"P={xw.tokens_per_frame} L={xw.text_tokens}",
                "layer_ms": round(f["layer"]["mean"], 4),
                "layer_median_ms": round(f["layer"]["median"], 4),
                "video_tokens_per_s": round(xw.batch * xw.video_tokens / (f["layer"]["mean"] / 1e3), 1),
                "softmax_ms": round(f["k1"]["mean"], 4),
                "softmax_frac_bf16_peak": round(xfl / (f["k1"]["mean"] / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "vda_ms": round(f["vda"]["mean"], 4),
                "vda_frac_hbm": round(vda_bytes(xw) / (f["vda"]["mean"] / 1e3) / 1e9 / PEAK_HBM_GBS, 4)}
        torch.cuda.empty_cache()
        extra["fp32_4h_20f"] = fp32_figures(max(5, args.steps // 4), 2)

    video_tokens = w.batch * w.video_tokens
    value = video_tokens / (ms / 1e3)
    k1_flops = softmax_flops(w)
    achieved = k1_flops / (k1_ms / 1e3) / 1e12
    vbytes = vda_bytes(w)
    lt = head["layer"]
    result = {
        "metric": "hybrid-attn layer ms & video tokens/s at 768p shape; % MFMA/HBM roofline",
        "value": round(value, 1),
        "unit": "video tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded, 768p-shaped: 24x42 latent grid per frame)",
        "config": {"workload": f"{w.name}: B={w.batch} H={w.heads} d={w.head_dim} "
                               f"T={w.frames} P={w.tokens_per_frame} L={w.text_tokens} "
                               f"chunk={w.chunk_frames} window=+-{w.window_chunks}",
                   "video_tokens": video_tokens, "parallelism": "single GPU"},
        "layer_ms": {"warm_mean": round(lt["mean"], 4), "warm_median": round(lt["median"], 4),
                     "warm_min": round(lt["min"], 4), "cold_median": round(lt["cold_median"], 4),
                     "cold_min": round(lt["cold_min"], 4),
                     "cold": "a 512 MiB write between calls (evicts L2 and MALL); events "
                             "around the layer call only"},
        "roofline": {"kernel": "softmax_vt_kernel<128, 1> (softmax + merge; the layer's second "
                               "stage, launched alone)",
                     "bound": "mfma",
                     "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(),
                     "algorithmic_flops_per_launch": k1_flops, "ms_per_launch": round(k1_ms, 4)},
        "vda": {"kernels": "vda_stats_kernel<128> + scan_split_kernel<128> + combine_kernel "
                           "(the layer's first stage, launched alone)",
                "bound": "hbm", "ms": round(vda_ms, 4), "algorithmic_bytes": vbytes,
                "achieved_gbs": round(vbytes / (vda_ms / 1e3) / 1e9, 1), "peak_gbs": PEAK_HBM_GBS,
                "frac": round(vbytes / (vda_ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
                "traffic": measured_traffic(VDA_TRAFFIC_FILE, VDA_SOURCES)},
        "other_workloads": extra or None,
        "wall_s_timed_region": round(head["wall"], 3),
        "output_projections": proj,
        "backward": bwd,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, inp)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
