#!/usr/bin/env python3
"""Benchmark of one Video DeltaNet hybrid video-to-video attention layer
forward on one MI355X, at the 768p shape (B=1, H=24, d=128, 60 latent frames x
1008 tokens = 60,480 video tokens, 512 text tokens, bf16).

A step is one call of the whole layer (vdn_hybrid_attn_fwd: Gram/write,
factor, scan, then the block-sparse softmax with the merge fused into its
epilogue) on synthetic inputs already resident in HBM.  Prints one JSON line:
layer throughput in video tokens/s, the roofline of the dominant kernel (the
fused softmax + merge stage, timed alone with HIP events on its stream), and
the CPU oracle timed on a bounded sample of the same workload.  It also times
the layer followed by the two branches' separate output projections
(d_model = H*d), the projection product alone, and the library matmul on the
same operands for comparison, and the backward pass (gradients of every input
given an upstream gradient of O).
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k1_softmax_768p_hbm_traffic.md")
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


def measured_traffic():
    """HBM bytes per softmax launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel sources; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].split(": ", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("sources_sha256_16") != sources_hash(K1_SOURCES):
        return None
    try:
        return int(float(vals["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, inp, budget_s=15.0):
    """The float64 oracle on a bounded sample: every token of five frames
    (both anchors and three interior frames), head after head of batch 0,
    until about budget_s seconds of CPU work (at least one head)."""
    from threadpoolctl import threadpool_info

    from oracle import vdn_oracle as O
    from video_diffusion_hybrid_block_amd import synth
    lay = O.Layout(**synth.layout_kwargs(w))
    frames = sorted({0, w.frames // 4, w.frames // 2, (3 * w.frames) // 4, w.frames - 1})
    P = w.tokens_per_frame
    import numpy as np
    tokens = np.concatenate([np.arange(f * P, (f + 1) * P) for f in frames])
    t0 = time.perf_counter()
    heads = 0
    while heads < w.heads:
        O.hybrid_attn_rows(inp, lay, 0, heads, tokens)
        heads += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    # one video token of the layer = all heads of that token
    tok_equiv = len(tokens) * heads / w.heads
    return {"value": tok_equiv / dt, "unit": "video tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{len(tokens)} query tokens (frames {frames}) x {heads} of {w.heads} heads, "
                      f"batch 0; {dt:.1f} s; counted as {len(tokens)}*{heads}/{w.heads} "
                      f"layer tokens"}


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
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(the layer shards by head; see the design notes). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from video_diffusion_hybrid_block_amd import binding as V
    from video_diffusion_hybrid_block_amd import synth

    w = synth.WORKLOADS[args.workload]
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
    o_fused = torch.empty_like(dev["q"])
    tk, tv = (dev["text_k"], dev["text_v"]) if L else (None, None)
    # the summed VDA states the fused stage reads (computed once, untimed)
    A, Bm = V.vda_gram(dev["k"], dev["v"], tk, tv, dev["beta"], **geo)
    R = V.vda_factor_scan(A, Bm, dev["alpha"], dtype=w.dtype, text_tokens=L, **geo)
    sws = torch.empty(max(V.softmax_workspace_size(lay), 1), dtype=torch.uint8, device="cuda")

    def layer():
        V.hybrid_attn(dev["q"], dev["k"], dev["v"], tk, tv, dev["beta"], dev["alpha"],
                      dev["gate_logits"], **geo, out=out, workspace=ws)

    def fused_stage():
        V.softmax_merge_fwd(dev["q"], dev["k"], dev["v"], tk, tv, R, dev["gate_logits"], **geo,
                            out=o_fused, workspace=sws)

    stream = torch.cuda.current_stream()
    print(f"[bench] warmup {args.warmup}, timing {args.steps} layer steps", file=sys.stderr,
          flush=True)
    for _ in range(args.warmup):
        layer()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        layer()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / args.steps

    # dominant kernel alone, same stream, same launch configuration (the
    # stage also runs the V^T copy that feeds it: ~1% of its time)
    for _ in range(2):
        fused_stage()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        fused_stage()
    e1.record(stream)
    torch.cuda.synchronize()
    k1_ms = e0.elapsed_time(e1) / args.steps

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
            "note": "vdn_hybrid_attn_fwd_train + vdn_hybrid_attn_bwd_saved: forward (same "
                    "output) keeping O_soft, RMSNorm(R q), lse, 1/r and the scan states; "
                    "backward from them; 14d flops per visible pair over the pair"}
        del saved, o_t, dO

    if args.copy_calib:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    video_tokens = w.batch * w.video_tokens
    value = video_tokens / (ms / 1e3)
    k1_flops = softmax_flops(w)
    achieved = k1_flops / (k1_ms / 1e3) / 1e12
    traffic = measured_traffic()
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
        "roofline": {"kernel": "softmax_vt_kernel<128, 1> (merge fused; + vt_transpose pre-pass)",
                     "bound": "mfma",
                     "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "algorithmic_flops_per_launch": k1_flops, "ms_per_launch": round(k1_ms, 4)},
        "wall_s_timed_region": round(wall, 3),
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
