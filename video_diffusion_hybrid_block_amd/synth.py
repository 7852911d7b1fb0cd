"""Seeded synthetic inputs for the hybrid video attention layer.

This module only draws random numbers and rounds them to the storage dtype; it
holds none of the layer's arithmetic.  The same arrays feed the HIP library
(through the binding) and the CPU oracle in the tests.

Shapes follow the pages' 768p workload: a 1344x768 video is a 24x42 latent grid
(1008 tokens per latent frame) and latent frames come in chunks of five
(PaperDaily explainer "伯克利与Impossible视频生成", §二 and §六).

Draw order (one ``numpy.random.default_rng(seed)`` stream, float64 draws):
q, k, v, text_k, text_v, beta, alpha, gate_logits.  Values are rounded to the
workload dtype (bf16 by round-to-nearest-even) and returned as float32 arrays
whose values are exactly representable in that dtype.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_inputs", "make_proj_weight", "make_gemm_operands",
           "round_bf16", "layout_kwargs"]


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    head_dim: int
    frames: int
    tokens_per_frame: int
    text_tokens: int
    dtype: str                 # "f32" | "bf16"
    seed: int
    beta_range: tuple | None = None    # None -> sigmoid(N(0,1)); else U[lo, hi]
    alpha_range: tuple = (0.9, 1.0)
    lowrank_keys: int = 0      # >0: keys of rank r per (batch, frame, head) + 1e-3 noise
    dup_fraction: float = 0.0  # share of tokens per frame overwritten by copies
    chunk_frames: int = 5
    window_chunks: int = 1

    @property
    def video_tokens(self) -> int:
        return self.frames * self.tokens_per_frame


# The five layer shapes.  Seeds are 1000 + the index in this list.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 1, 16, 20, 16, 8, "f32", 1000),
    "small_bf16": Workload("small_bf16", 1, 8, 64, 30, 112, 64, "bf16", 1001),
    "768p": Workload("768p", 1, 24, 128, 60, 1008, 512, "bf16", 1002),
    "long_120f": Workload("long_120f", 1, 24, 128, 120, 1008, 512, "bf16", 1003),
    "stress_lowrank": Workload("stress_lowrank", 2, 24, 128, 60, 1008, 512, "bf16", 1004,
                               beta_range=(0.01, 10.0), alpha_range=(0.5, 1.0),
                               lowrank_keys=8, dup_fraction=0.25),
}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even); returns float32."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    r = ((u + bias) & np.uint32(0xFFFF0000)).astype(np.uint32)
    return r.view(np.float32)


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return round_bf16(x) if dtype == "bf16" else x


def _unit_rows(x: np.ndarray) -> np.ndarray:
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def layout_kwargs(w: Workload) -> dict:
    """Keyword arguments shared by the oracle's Layout and the binding."""
    return dict(batch=w.batch, heads=w.heads, head_dim=w.head_dim, frames=w.frames,
                tokens_per_frame=w.tokens_per_frame, text_tokens=w.text_tokens,
                chunk_frames=w.chunk_frames, window_chunks=w.window_chunks)


def _lowrank_keys(rng, w: Workload):
    """Per (batch, frame, head): an orthonormal d x r basis U (QR of a Gaussian),
    keys U c + 1e-3 noise, then a share of tokens replaced by copies of other
    tokens of the same frame (keys and values together)."""
    B, T, P, H, d, r = w.batch, w.frames, w.tokens_per_frame, w.heads, w.head_dim, w.lowrank_keys
    k = np.empty((B, T, P, H, d), dtype=np.float64)
    for b in range(B):
        for t in range(T):
            for h in range(H):
                U, _ = np.linalg.qr(rng.standard_normal((d, r)))
                c = rng.standard_normal((P, r))
                k[b, t, :, h] = c @ U.T + 1e-3 * rng.standard_normal((P, d))
    return k


def make_inputs(w: Workload | str, seed: int | None = None) -> dict:
    """Arrays (float32, values exact in the workload dtype):
    q, k, v [B, T*P, H, d]; text_k, text_v [B, L, H, d];
    beta [B, T*P + L, H]; alpha [B, T, H]; gate_logits [B, T*P, H, 2]."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = np.random.default_rng(w.seed if seed is None else seed)
    B, H, d, T, P, L = w.batch, w.heads, w.head_dim, w.frames, w.tokens_per_frame, w.text_tokens
    N = T * P
    q = _cast(rng.standard_normal((B, N, H, d)), w.dtype)
    if w.lowrank_keys:
        k_raw = _lowrank_keys(rng, w)                       # [B, T, P, H, d]
        v5 = rng.standard_normal((B, T, P, H, d))
        n_dup = int(round(w.dup_fraction * P))
        for b in range(B):
            for t in range(T):
                for h in range(H):
                    perm = rng.permutation(P)
                    dst, pool = perm[:n_dup], perm[n_dup:]
                    src = pool[rng.integers(0, len(pool), size=n_dup)]
                    k_raw[b, t, dst, h] = k_raw[b, t, src, h]
                    v5[b, t, dst, h] = v5[b, t, src, h]
        k = _cast(_unit_rows(k_raw).reshape(B, N, H, d), w.dtype)
        v = _cast(v5.reshape(B, N, H, d), w.dtype)
        del k_raw, v5
    else:
        k = _cast(_unit_rows(rng.standard_normal((B, N, H, d))), w.dtype)
        v = _cast(rng.standard_normal((B, N, H, d)), w.dtype)
    text_k = _cast(_unit_rows(rng.standard_normal((B, L, H, d))), w.dtype)
    text_v = _cast(rng.standard_normal((B, L, H, d)), w.dtype)
    if w.beta_range is None:
        beta = _sigmoid(rng.standard_normal((B, N + L, H)))
    else:
        beta = rng.uniform(w.beta_range[0], w.beta_range[1], size=(B, N + L, H))
    alpha = rng.uniform(w.alpha_range[0], w.alpha_range[1], size=(B, T, H))
    gates = rng.standard_normal((B, N, H, 2))
    return dict(q=q, k=k, v=v, text_k=text_k, text_v=text_v,
                beta=beta.astype(np.float32), alpha=alpha.astype(np.float32),
                gate_logits=gates.astype(np.float32))


def make_proj_weight(d_model: int, heads: int, head_dim: int, seed: int,
                     dtype: str = "bf16") -> np.ndarray:
    """Output-projection weights w_o [d_model, 2*H*d] in (out, in) order,
    softmax-branch input columns first: N(0, 1 / (2*H*d)) draws (a random
    initialisation of a trained projection's scale), rounded to dtype;
    float32 array."""
    rng = np.random.default_rng(seed)
    K = 2 * heads * head_dim
    return _cast(rng.standard_normal((d_model, K)) / np.sqrt(K), dtype)


def make_gemm_operands(M: int, K: int, N: int, seed: int) -> tuple:
    """x [M, K] ~ N(0, 1) and w [N, K] ~ N(0, 1/K), both rounded to bf16
    (float32 arrays), for the projection product on its own."""
    rng = np.random.default_rng(seed)
    x = _cast(rng.standard_normal((M, K)), "bf16")
    w = _cast(rng.standard_normal((N, K)) / np.sqrt(K), "bf16")
    return x, w
