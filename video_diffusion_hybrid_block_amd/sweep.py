"""Dense vs hybrid softmax across video lengths (42 -> 102 latent frames).

The softmax kernel takes any window: with ``window_chunks`` at least the
number of chunks every frame sees every frame, which is plain dense attention
over video + text keys.  This sweep times, per frame count, on the 768p
frame shape (24 heads, d = 128, 1008 tokens per frame, 512 text tokens, bf16):

- the hybrid layer (``vdn_hybrid_attn_fwd``),
- the hybrid softmax stage (chunks of 5, own chunk +- 1, two anchor frames),
- the dense softmax stage (window covering the whole video),

and reports the softmax density the hybrid mask keeps (share of video
(query frame, key frame) pairs, the figure the PaperDaily explainer §七 quotes
for 42 and 102 latent frames), the increment the anchors add to it (the
deepmagic blog, section 用兩條分支取代一條, and the aimodeling article,
"The VDN split", print 3.57 %), and the measured dense / hybrid time ratio.

Inputs are synthetic, drawn on the device from a seeded generator with the
768p workload's distributions (q, v ~ N(0,1); k ~ N(0,1) L2-normalised;
beta = sigmoid(N(0,1)); alpha ~ U[0.9, 1); gate logits ~ N(0,1)).

    python -m video_diffusion_hybrid_block_amd.sweep [--frames 42 60 81 102] [--reps 5]

``--tiles-only`` prints the same densities at the kernel's own granularity
(256-query work items x 64-key tiles, partial tiles counted whole) without
touching the GPU.
"""
from __future__ import annotations

import argparse
import json
import sys


def visible_frame_counts(frames: int, chunk: int, window: int, anchors: bool) -> list[int]:
    """Number of key frames each query frame's softmax sees (anchor frames see
    every frame; the others their chunk window plus the anchors)."""
    out = []
    for t in range(frames):
        if anchors and t in (0, frames - 1):
            out.append(frames)
            continue
        c = t // chunk
        lo, hi = max(0, (c - window) * chunk), min(frames, (c + window + 1) * chunk)
        vis = set(range(lo, hi))
        if anchors:
            vis |= {0, frames - 1}
        out.append(len(vis))
    return out


def density(frames: int, chunk: int = 5, window: int = 1, anchors: bool = True) -> float:
    """Share of video (query frame, key frame) pairs the softmax handles."""
    return sum(visible_frame_counts(frames, chunk, window, anchors)) / float(frames * frames)


# Work item of the softmax kernel: 256 queries of one frame against its
# visible keys (the window's frames, the anchors, then the text), packed
# back to back and taken 64 keys at a time.
ITEM_QUERIES, TILE_KEYS = 256, 64


def tile_count(frames: int, P: int, L: int, chunk: int = 5, window: int = 1,
               anchors: bool = True, text: bool = True) -> int:
    """(256-query item, 64-key tile) pairs the softmax kernel runs for one
    head: every frame has ceil(P / 256) items, each with ceil(n / 64) key
    tiles for its n visible keys (text keys counted when `text`)."""
    items = -(-P // ITEM_QUERIES)
    return sum(items * (-(-(v * P + (L if text else 0)) // TILE_KEYS))
               for v in visible_frame_counts(frames, chunk, window, anchors))


def tile_density(frames: int, P: int, L: int, chunk: int = 5, window: int = 1,
                 anchors: bool = True, text: bool = False) -> float:
    """The softmax density at the kernel's granularity: its (item, key tile)
    pairs over those of dense attention on the same frames (a window that
    covers every chunk), video keys only unless `text`."""
    nc = -(-frames // chunk)
    return (tile_count(frames, P, L, chunk, window, anchors, text)
            / float(tile_count(frames, P, L, chunk, nc, anchors, text)))


def tile_rows(frame_counts, P: int = 1008, L: int = 512, chunk: int = 5, window: int = 1):
    """Frame-pair and tile-granularity density and anchor increment per frame
    count (no GPU)."""
    rows = []
    for T in frame_counts:
        row = {"frames": T,
               "density_pct": round(100 * density(T, chunk, window, True), 3),
               "anchor_increment_pct": round(100 * (density(T, chunk, window, True)
                                                    - density(T, chunk, window, False)), 3)}
        for text in (False, True):
            tag = "_with_text" if text else ""
            a = tile_density(T, P, L, chunk, window, True, text)
            na = tile_density(T, P, L, chunk, window, False, text)
            row[f"tile_density{tag}_pct"] = round(100 * a, 3)
            row[f"tile_anchor_increment{tag}_pct"] = round(100 * (a - na), 3)
        rows.append(row)
    return rows


def softmax_flops(frames: int, P: int, L: int, H: int, d: int, chunk: int, window: int) -> float:
    """4*d flops per visible (query, key) pair, text keys included."""
    vis = visible_frame_counts(frames, chunk, window, True)
    pairs = sum(v * P + L for v in vis) * P
    return 4.0 * d * pairs * H


def make_inputs(frames, P, L, H, d, seed, device="cuda"):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    N = frames * P

    def randn(*shape):
        return torch.randn(*shape, generator=g, device=device, dtype=torch.float32)

    k = randn(1, N, H, d)
    k = k / k.norm(dim=-1, keepdim=True)
    tk = randn(1, L, H, d)
    tk = tk / tk.norm(dim=-1, keepdim=True)
    inp = {
        "q": randn(1, N, H, d).to(torch.bfloat16),
        "k": k.to(torch.bfloat16),
        "v": randn(1, N, H, d).to(torch.bfloat16),
        "text_k": tk.to(torch.bfloat16),
        "text_v": randn(1, L, H, d).to(torch.bfloat16),
        "beta": torch.sigmoid(randn(1, N + L, H)).contiguous(),
        "alpha": (0.9 + 0.1 * torch.rand(1, frames, H, generator=g, device=device)).contiguous(),
        "gate_logits": randn(1, N, H, 2),
    }
    return inp


def time_call(fn, reps, warmup=1):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--frames", type=int, nargs="+", default=[42, 60, 81, 102])
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--tokens-per-frame", type=int, default=1008)
    ap.add_argument("--text-tokens", type=int, default=512)
    ap.add_argument("--heads", type=int, default=24)
    ap.add_argument("--json", action="store_true", help="one JSON object per frame count")
    ap.add_argument("--tiles-only", action="store_true",
                    help="print the frame-pair and tile-granularity densities only (no GPU)")
    args = ap.parse_args(argv)

    if args.tiles_only:
        rows = tile_rows(args.frames, args.tokens_per_frame, args.text_tokens)
        if args.json:
            for r in rows:
                print(json.dumps(r))
            return
        print("| frames | density (frame pairs) | anchor incr. (frame pairs) | density (tiles) | "
              "anchor incr. (tiles) | density (tiles, text keys incl.) | "
              "anchor incr. (tiles, text keys incl.) |")
        print("|" + "---|" * 7)
        for r in rows:
            print(f"| {r['frames']} | {r['density_pct']} % | {r['anchor_increment_pct']} % | "
                  f"{r['tile_density_pct']} % | {r['tile_anchor_increment_pct']} % | "
                  f"{r['tile_density_with_text_pct']} % | "
                  f"{r['tile_anchor_increment_with_text_pct']} % |")
        return

    import torch

    from . import binding as V

    P, L, H, d, C, W = args.tokens_per_frame, args.text_tokens, args.heads, 128, 5, 1
    rows = []
    for T in args.frames:
        print(f"[sweep] {T} frames: generating inputs", file=sys.stderr, flush=True)
        inp = make_inputs(T, P, L, H, d, seed=2000 + T)
        nc = (T + C - 1) // C
        geo_h = dict(frames=T, tokens_per_frame=P, chunk_frames=C, window_chunks=W)
        geo_d = dict(frames=T, tokens_per_frame=P, chunk_frames=C, window_chunks=nc)
        out = torch.empty_like(inp["q"])
        o2 = torch.empty_like(inp["q"])
        lay = V.make_layout(batch=1, heads=H, head_dim=d, frames=T, tokens_per_frame=P,
                            text_tokens=L, dtype="bf16", chunk_frames=C, window_chunks=W)
        ws = torch.empty(V.workspace_size(lay), dtype=torch.uint8, device="cuda")
        sws = torch.empty(max(V.softmax_workspace_size(lay), 1), dtype=torch.uint8, device="cuda")

        def layer():
            V.hybrid_attn(inp["q"], inp["k"], inp["v"], inp["text_k"], inp["text_v"], inp["beta"],
                          inp["alpha"], inp["gate_logits"], **geo_h, out=out, workspace=ws)

        def soft_h():
            V.softmax_fwd(inp["q"], inp["k"], inp["v"], inp["text_k"], inp["text_v"], **geo_h,
                          out=o2, workspace=sws)

        def soft_d():
            V.softmax_fwd(inp["q"], inp["k"], inp["v"], inp["text_k"], inp["text_v"], **geo_d,
                          out=o2, workspace=sws)

        t_layer = time_call(layer, args.reps)
        t_h = time_call(soft_h, args.reps)
        t_d = time_call(soft_d, args.reps)
        f_h = softmax_flops(T, P, L, H, d, C, W)
        f_d = softmax_flops(T, P, L, H, d, C, nc)
        row = {
            "frames": T, "video_tokens": T * P,
            "density_pct": round(100 * density(T, C, W, True), 2),
            "density_no_anchor_pct": round(100 * density(T, C, W, False), 2),
            "anchor_increment_pct": round(100 * (density(T, C, W, True) - density(T, C, W, False)), 3),
            "layer_ms": round(t_layer, 3), "video_tokens_per_s": round(T * P / (t_layer / 1e3), 1),
            "softmax_hybrid_ms": round(t_h, 3), "softmax_dense_ms": round(t_d, 3),
            "dense_over_hybrid": round(t_d / t_h, 3),
            "hybrid_tflops": round(f_h / (t_h / 1e3) / 1e12, 1),
            "dense_tflops": round(f_d / (t_d / 1e3) / 1e12, 1),
        }
        rows.append(row)
        if args.json:
            print(json.dumps(row), flush=True)
        del inp, out, o2, ws, sws
        torch.cuda.empty_cache()

    if not args.json:
        hdr = ("| frames | video tokens | density | anchor incr. | hybrid layer ms | layer tok/s | "
               "softmax hybrid ms | softmax dense ms | dense / hybrid | hybrid TFLOP/s | dense TFLOP/s |")
        print(hdr)
        print("|" + "---|" * 11)
        for r in rows:
            print(f"| {r['frames']} | {r['video_tokens']} | {r['density_pct']} % | "
                  f"{r['anchor_increment_pct']} % | {r['layer_ms']} | {r['video_tokens_per_s']:.3e} | "
                  f"{r['softmax_hybrid_ms']} | {r['softmax_dense_ms']} | {r['dense_over_hybrid']} | "
                  f"{r['hybrid_tflops']} | {r['dense_tflops']} |")


if __name__ == "__main__":
    main()
