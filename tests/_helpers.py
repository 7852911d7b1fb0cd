"""Shared helpers for the parity tests: device transfer, oracle layouts and
error metrics (relative Frobenius error, the tolerance metric of the tests)."""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

from oracle import vdn_oracle as O
from video_diffusion_hybrid_block_amd import synth

# Output tolerances: relative Frobenius error of O against the oracle.
TOL = {"f32": 1e-4, "bf16": 2e-2}


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from video_diffusion_hybrid_block_amd import binding
    binding.lib()   # must load on a GPU machine: no fallback


def workload(name, **over) -> synth.Workload:
    return dataclasses.replace(synth.WORKLOADS[name], **over) if over else synth.WORKLOADS[name]


def custom(name, *, batch, heads, head_dim, frames, tokens_per_frame, text_tokens, dtype,
           seed=7, chunk_frames=5, window_chunks=1, **kw) -> synth.Workload:
    return synth.Workload(name, batch, heads, head_dim, frames, tokens_per_frame, text_tokens,
                          dtype, seed, chunk_frames=chunk_frames, window_chunks=window_chunks, **kw)


def oracle_layout(w: synth.Workload, **over) -> O.Layout:
    kw = synth.layout_kwargs(w)
    kw.update(over)
    return O.Layout(**kw)


def to_dev(inp: dict, dtype: str) -> dict:
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = {}
    for key, arr in inp.items():
        t = torch.from_numpy(np.ascontiguousarray(arr))
        if key in ("q", "k", "v", "text_k", "text_v"):
            t = t.to(tdt)
        out[key] = t.cuda()
    return out


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def sample_tokens(w: synth.Workload, rng) -> np.ndarray:
    """Tokens spanning anchor, edge and interior frames, and inside every
    frame both sides of each 256-query work-item edge of the softmax kernel
    (255/256, 511/512, 767/768), the 32-query wave edges (31/32), the start of
    the ragged last item (P - 240 at P = 1008) and the frame's last rows."""
    T, P = w.frames, w.tokens_per_frame
    frames = sorted({f for f in (0, 1, 4, 5, 9, 10, T // 2, T - 6, T - 5, T - 2, T - 1) if 0 <= f < T})
    local = {0, 1, 31, 32, 255, 256, 511, 512, 767, 768, P - 240, P - 113, P - 33, P - 2, P - 1}
    local |= set(rng.integers(0, P, size=4).tolist())
    local = sorted(x for x in local if 0 <= x < P)
    return np.array([f * P + x for f in frames for x in local], dtype=np.int64)


def oracle_chunk_reads(inp: dict, lay, w: synth.Workload) -> np.ndarray:
    """R [B, H, nc+1, d, d] float32 from the oracle's per-frame states: slot c
    holds what the non-anchor frames of chunk c read (taken from the chunk's
    first non-anchor frame; zero when the chunk holds anchors only), slot nc
    the text write (what an anchor frame reads)."""
    nc = lay.num_chunks
    d = w.head_dim
    anchors = set(O.anchor_frames(lay))
    R = np.zeros((w.batch, w.heads, nc + 1, d, d), np.float32)
    for b in range(w.batch):
        for h in range(w.heads):
            per_frame = O.chunk_states(inp["k"], inp["v"], inp["text_k"], inp["text_v"], inp["beta"],
                                       inp["alpha"], lay, b, h)
            for c in range(nc):
                frames = [t for t in range(c * lay.chunk_frames,
                                           min((c + 1) * lay.chunk_frames, w.frames))
                          if t not in anchors]
                if frames:
                    R[b, h, c] = per_frame[frames[0]]
            R[b, h, nc] = per_frame[min(anchors)] if anchors else 0.0
    return R


def max_abs_ratio(got, ref) -> float:
    """max |got - ref| / max |ref| (reported beside the Frobenius metric)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


def write_parity_summary(name: str, record: dict) -> None:
    """Append one JSON line per checked configuration to the file the
    environment variable VDN_PARITY_SUMMARY names (nothing if it is unset)."""
    import json
    import os
    path = os.environ.get("VDN_PARITY_SUMMARY")
    if not path:
        return
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "a") as fh:
        fh.write(json.dumps({"config": name, **record}) + "\n")
