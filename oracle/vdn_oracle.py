"""Plain, slow float64 CPU oracle for the Video DeltaNet hybrid video-to-video
attention layer (one layer, forward).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The HIP library
and its Python binding never import it and share no code with it.

Every function is the definition written out, in the pages' order, with numpy
float64 and a library SPD solve as the only primitives.  Sources (cited by page
title and section):

* [PD]  PaperDaily explainer "伯克利与Impossible视频生成:14.3秒视频6.70秒去噪"
        (longzhangge.com), sections 二 (近处精看,远处记住), 三 (同时向前看,
        也向后看), 四 (整帧一起写) with its pseudocode block, 七.
* [ABS] arXiv listing "Video DeltaNet: A Video-Native Hybrid Attention for
        Livestream Video Generation", English abstract.
* [DM]  deepmagic blog "生成比播放還快：Video DeltaNet 用 11 秒產出 14 秒 768p
        影片", section 用兩條分支取代一條 (closed form S=(S̄+B)(I+A)^-1).
* [AM]  aimodeling article "Video DeltaNet Makes H3 Video Generation Faster
        Than Playback", section "The VDN split: local Softmax plus long-range
        linear memory".

Readings where the pages are silent (each is a keyword argument of
``Readings``; the GPU implements only the primary value):

* R1  softmax scale 1/sqrt(d_k).
* R2  chunks of ``chunk_frames`` counted from frame 0, last chunk may be
      partial, window = own chunk +- ``window_chunks``, clipped at the ends.
* R3  anchors inside the window are counted once (set union).
* R4  one softmax over video keys of visible frames together with all text
      keys; only video tokens are queries.
* R5  anchor query frames have no far frames, so both states stay at the
      half text write and the linear read is the whole text write
      (``anchor_read="text_prior"``; alternative ``"zero"``).
* R6  anchor frames are skipped by the scan entirely: no write, no decay
      (``anchor_decay=False``; alternative True = decay without write).
* R7  half text write = 0.5 * B_x (I + A_x)^-1, the update from the zero state
      (``half_write="vda"``; alternative ``"raw"`` = 0.5 * B_x).
* R8  one decay alpha per (batch, frame, head), shared by both directions.
* R9  q and k enter the linear branch as given (no feature map).
* R10 one gate logit per (batch, token, head, branch).
* R11 RMSNorm epsilon 1e-6, no learnable weight.
* R12 no output projection: O is the gated sum per head.
* R13 one beta tensor covering video tokens then text tokens.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
from scipy.linalg import cho_factor, cho_solve

__all__ = [
    "Layout", "Readings", "PRIMARY",
    "chunk_of", "window_frames", "anchor_frames", "visible_frames",
    "far_forward", "far_backward", "pair_class", "softmax_density",
    "softmax_rows", "softmax_branch", "frame_stats", "vda_update",
    "text_prior", "initial_state", "forward_state", "backward_state",
    "linear_read_rows", "rms_norm", "merge", "hybrid_attn_rows",
    "hybrid_attn", "chunk_states",
]


@dataclass(frozen=True)
class Layout:
    """Shape and geometry of one layer call (tensors are [B, tokens, H, d])."""
    batch: int
    heads: int
    head_dim: int
    frames: int
    tokens_per_frame: int
    text_tokens: int
    chunk_frames: int = 5
    window_chunks: int = 1
    anchor_first: bool = True
    anchor_last: bool = True
    softmax_scale: float = 0.0   # 0 -> 1/sqrt(d)   (R1)
    rms_eps: float = 1e-6        # (R11)

    @property
    def video_tokens(self) -> int:
        return self.frames * self.tokens_per_frame

    @property
    def num_chunks(self) -> int:
        return -(-self.frames // self.chunk_frames)

    @property
    def scale(self) -> float:
        return self.softmax_scale if self.softmax_scale > 0 else 1.0 / np.sqrt(self.head_dim)


@dataclass(frozen=True)
class Readings:
    anchor_read: str = "text_prior"   # R5
    anchor_decay: bool = False        # R6
    half_write: str = "vda"           # R7


PRIMARY = Readings()


# ---------------------------------------------------------------------------
# Frame-level geometry  [PD §二; DM 用兩條分支取代一條; AM "The VDN split"]
# ---------------------------------------------------------------------------

def chunk_of(lay: Layout, t: int) -> int:
    """Latent frames are grouped into consecutive chunks of ``chunk_frames``
    (five in the pages, the video encoder's temporal unit) [PD §二]."""
    return t // lay.chunk_frames


def window_frames(lay: Layout, t: int) -> list[int]:
    """A query chunk sees its own chunk and the neighbouring chunks
    (``window_chunks`` = 1: previous and next) [PD §二; AM "The VDN split"]."""
    ct = chunk_of(lay, t)
    return [f for f in range(lay.frames)
            if abs(chunk_of(lay, f) - ct) <= lay.window_chunks]


def anchor_frames(lay: Layout) -> set[int]:
    """Boundary anchors: the first and the last latent frame [PD §二;
    DM 用兩條分支取代一條 (4-way boundary anchors)]."""
    a = set()
    if lay.frames > 0 and lay.anchor_first:
        a.add(0)
    if lay.frames > 0 and lay.anchor_last:
        a.add(lay.frames - 1)
    return a


def visible_frames(lay: Layout, t: int) -> list[int]:
    """Key frames the softmax branch sees for query frame t: an anchor frame
    sees the whole sequence; any other frame sees its window plus the anchors
    (set union, R3) [PD §二; AM "The VDN split"]."""
    anchors = anchor_frames(lay)
    if t in anchors:
        return list(range(lay.frames))
    return sorted(set(window_frames(lay, t)) | anchors)


def far_forward(lay: Layout, t: int) -> list[int]:
    """Far frames before t, ascending: what the forward state summarises
    (everything before the local window that is not an anchor) [PD §三]."""
    vis = set(visible_frames(lay, t))
    return [f for f in range(t) if f not in vis]


def far_backward(lay: Layout, t: int) -> list[int]:
    """Far frames after t, descending: what the backward state summarises
    [PD §三]."""
    vis = set(visible_frames(lay, t))
    return [f for f in range(lay.frames - 1, t, -1) if f not in vis]


def pair_class(lay: Layout, t: int, f: int) -> str:
    """Class of the (query frame t, key frame f) pair: 'window' (local
    softmax), 'anchor' (softmax through a boundary anchor) or 'far' (linear
    memory) [PD §二, figure 2 description]."""
    if f in window_frames(lay, t):
        return "window"
    anchors = anchor_frames(lay)
    if f in anchors or t in anchors:
        return "anchor"
    return "far"


def softmax_density(lay: Layout, with_anchors: bool = True) -> float:
    """Share of video (query frame, key frame) pairs handled by softmax, for
    equal tokens per frame (the density the pages quote) [PD §七;
    DM 用兩條分支取代一條]."""
    T = lay.frames
    if not with_anchors:
        lay = Layout(**{**lay.__dict__, "anchor_first": False, "anchor_last": False})
    n = sum(len(visible_frames(lay, t)) for t in range(T))
    return n / float(T * T)


# ---------------------------------------------------------------------------
# Softmax branch  [PD §二; ABS; AM "The VDN split"]
# ---------------------------------------------------------------------------

def _frame_rows(lay: Layout, f: int) -> slice:
    P = lay.tokens_per_frame
    return slice(f * P, (f + 1) * P)


def softmax_rows(q, k, v, text_k, text_v, lay: Layout, b: int, h: int,
                 tokens) -> np.ndarray:
    """O_soft for the given video query tokens of (b, h): one softmax over the
    keys of the query frame's visible frames together with every text key
    (text interactions keep softmax, R4) [ABS; PD §二]."""
    tokens = np.asarray(tokens, dtype=np.int64)
    out = np.zeros((len(tokens), v.shape[-1]), dtype=np.float64)
    frames_of = tokens // lay.tokens_per_frame
    for t in np.unique(frames_of):
        sel = np.nonzero(frames_of == t)[0]
        kf = [np.asarray(k[b, _frame_rows(lay, f), h], np.float64) for f in visible_frames(lay, int(t))]
        vf = [np.asarray(v[b, _frame_rows(lay, f), h], np.float64) for f in visible_frames(lay, int(t))]
        if lay.text_tokens > 0:
            kf.append(np.asarray(text_k[b, :, h], np.float64))
            vf.append(np.asarray(text_v[b, :, h], np.float64))
        K = np.concatenate(kf, axis=0)
        V = np.concatenate(vf, axis=0)
        Q = np.asarray(q[b, tokens[sel], h], np.float64)
        s = (Q @ K.T) * lay.scale
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[sel] = p @ V
    return out


def softmax_branch(q, k, v, text_k, text_v, lay: Layout) -> np.ndarray:
    """O_soft for every video token of every (b, h)."""
    out = np.zeros(q.shape, dtype=np.float64)
    all_tokens = np.arange(lay.video_tokens)
    for b in range(lay.batch):
        for h in range(lay.heads):
            out[b, :, h] = softmax_rows(q, k, v, text_k, text_v, lay, b, h, all_tokens)
    return out


# ---------------------------------------------------------------------------
# Video Delta Attention  [DM 用兩條分支取代一條; PD §四; AM "The VDN split"]
# ---------------------------------------------------------------------------

def frame_stats(k_rows, v_rows, beta_rows):
    """Statistics of one frame's (k, v, beta) tokens: the key Gram
    A = sum_i beta_i k_i k_i^T (key correlation inside the frame) and the
    write B = sum_i beta_i v_i k_i^T [DM 用兩條分支取代一條; PD §四]."""
    k_rows = np.asarray(k_rows, np.float64)
    v_rows = np.asarray(v_rows, np.float64)
    beta_rows = np.asarray(beta_rows, np.float64)
    A = (k_rows * beta_rows[:, None]).T @ k_rows
    B = (v_rows * beta_rows[:, None]).T @ k_rows
    return A, B


def vda_update(S_bar, A, B):
    """The frame-wise joint update: the minimiser of
    ||S - S_bar||_F^2 + sum_i beta_i ||S k_i - v_i||^2, i.e.
    S = (S_bar + B)(I + A)^-1, computed with an SPD solve of (I + A) (never an
    explicit inverse) [DM 用兩條分支取代一條; PD §四]."""
    d = A.shape[0]
    M = np.eye(d) + A
    rhs = np.asarray(S_bar, np.float64) + B
    # S M = rhs  <=>  M S^T = rhs^T  (M symmetric positive definite)
    return cho_solve(cho_factor(M, lower=True), rhs.T).T


def text_prior(text_k, text_v, beta_text):
    """S_x: the text write, the joint update of all text tokens from the zero
    state (R7)."""
    A, B = frame_stats(text_k, text_v, beta_text)
    return vda_update(np.zeros_like(B), A, B)


def initial_state(text_k, text_v, beta_text, d_v, d_k, readings: Readings = PRIMARY):
    """Both states start from half of the text write, so the text counts once
    after the two reads are summed [PD §三; DM 用兩條分支取代一條 (×½)]."""
    if text_k is None or len(text_k) == 0:
        return np.zeros((d_v, d_k))
    if readings.half_write == "vda":
        return 0.5 * text_prior(text_k, text_v, beta_text)
    A, B = frame_stats(text_k, text_v, beta_text)
    return 0.5 * B


def _fold(S0, frames, stats, alpha_bh, decay_only=()):
    """Apply decay then the joint update for each frame in order (pseudocode
    steps 1-3 of PD §四).  ``decay_only`` frames only decay (reading R6 alt)."""
    S = S0.copy()
    for f in frames:
        if f in decay_only:
            S = alpha_bh[f] * S
            continue
        A, B = stats[f]
        S = vda_update(alpha_bh[f] * S, A, B)
    return S


def _scan_order(lay: Layout, t: int, direction: str, readings: Readings):
    far = far_forward(lay, t) if direction == "f" else far_backward(lay, t)
    if not readings.anchor_decay or not far:
        return far, ()
    # R6 alternative: anchors on the far side of the window decay the state.
    anchors = anchor_frames(lay)
    if direction == "f":
        lim = max(far)
        extra = [a for a in anchors if a < lim]
        order = sorted(set(far) | set(extra))
    else:
        lim = min(far)
        extra = [a for a in anchors if a > lim]
        order = sorted(set(far) | set(extra), reverse=True)
    return order, tuple(extra)


def _frame_stats_bh(k, v, beta, lay: Layout, b: int, h: int, frames):
    P = lay.tokens_per_frame
    stats = {}
    for f in frames:
        rows = _frame_rows(lay, f)
        stats[f] = frame_stats(k[b, rows, h], v[b, rows, h], beta[b, f * P:(f + 1) * P, h])
    return stats


def forward_state(S0, lay, t, stats, alpha_bh, readings: Readings = PRIMARY):
    """S^f(t): fold over the far frames before the window, ascending [PD §三]."""
    order, dec = _scan_order(lay, t, "f", readings)
    return _fold(S0, order, stats, alpha_bh, dec)


def backward_state(S0, lay, t, stats, alpha_bh, readings: Readings = PRIMARY):
    """S^b(t): fold over the far frames after the window, descending [PD §三]."""
    order, dec = _scan_order(lay, t, "b", readings)
    return _fold(S0, order, stats, alpha_bh, dec)


def _bh_states(k, v, text_k, text_v, beta, alpha, lay: Layout, b: int, h: int,
               frames_needed, readings: Readings):
    """(S^f(t), S^b(t)) for each query frame t in ``frames_needed``; every
    fold is recomputed from scratch (no shared prefix)."""
    d_k = k.shape[-1]
    d_v = v.shape[-1]
    N = lay.video_tokens
    L = lay.text_tokens
    if L > 0:
        S0 = initial_state(text_k[b, :, h], text_v[b, :, h], beta[b, N:N + L, h], d_v, d_k, readings)
    else:
        S0 = np.zeros((d_v, d_k))
    needed = set()
    for t in frames_needed:
        needed |= set(far_forward(lay, t)) | set(far_backward(lay, t))
    stats = _frame_stats_bh(k, v, beta, lay, b, h, sorted(needed))
    alpha_bh = np.asarray(alpha[b, :, h], np.float64)
    out = {}
    anchors = anchor_frames(lay)
    for t in frames_needed:
        if t in anchors and readings.anchor_read == "zero":
            out[t] = (np.zeros_like(S0), np.zeros_like(S0))
            continue
        out[t] = (forward_state(S0, lay, t, stats, alpha_bh, readings),
                  backward_state(S0, lay, t, stats, alpha_bh, readings))
    return out


def chunk_states(k, v, text_k, text_v, beta, alpha, lay: Layout, b: int, h: int,
                 readings: Readings = PRIMARY):
    """R(t) = S^f(t) + S^b(t) for every frame of (b, h), as a [T, d_v, d_k]
    array (used to check intermediate GPU results)."""
    st = _bh_states(k, v, text_k, text_v, beta, alpha, lay, b, h, range(lay.frames), readings)
    return np.stack([st[t][0] + st[t][1] for t in range(lay.frames)])


def rms_norm(o, eps):
    """RMS normalisation of the linear read over its channels, no weight
    (R11) [PD §三]."""
    return o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def merge(o_soft, n_lin, gate_logits):
    """Content-dependent sigmoid gates calibrate each branch before the sum
    (R10, R12) [PD §三; DM 用兩條分支取代一條]."""
    g = np.asarray(gate_logits, np.float64)
    return _sigmoid(g[..., 0:1]) * o_soft + _sigmoid(g[..., 1:2]) * n_lin


def linear_read_rows(q, states, lay: Layout, b: int, h: int, tokens):
    """o_i = (S^f(t) + S^b(t)) q_i, the sum of the two reads [PD §三]."""
    tokens = np.asarray(tokens, dtype=np.int64)
    Q = np.asarray(q[b, tokens, h], np.float64)
    out = np.zeros((len(tokens), states[next(iter(states))][0].shape[0]))
    frames_of = tokens // lay.tokens_per_frame
    for i, t in enumerate(frames_of):
        Sf, Sb = states[int(t)]
        out[i] = (Sf + Sb) @ Q[i]
    return out


def hybrid_attn_rows(inputs: dict, lay: Layout, b: int, h: int, tokens,
                     readings: Readings = PRIMARY, parts: bool = False):
    """Layer output O for the given video tokens of (b, h).  ``inputs`` holds
    q, k, v, text_k, text_v, beta, alpha, gate_logits (see ``hybrid_attn``).
    With ``parts`` returns (O, O_soft, o_lin, n_lin)."""
    q, k, v = inputs["q"], inputs["k"], inputs["v"]
    tk, tv = inputs["text_k"], inputs["text_v"]
    beta, alpha, gates = inputs["beta"], inputs["alpha"], inputs["gate_logits"]
    tokens = np.asarray(tokens, dtype=np.int64)
    o_soft = softmax_rows(q, k, v, tk, tv, lay, b, h, tokens)
    frames = sorted(set((tokens // lay.tokens_per_frame).tolist()))
    states = _bh_states(k, v, tk, tv, beta, alpha, lay, b, h, frames, readings)
    o_lin = linear_read_rows(q, states, lay, b, h, tokens)
    n_lin = rms_norm(o_lin, lay.rms_eps)
    out = merge(o_soft, n_lin, np.asarray(gates[b, tokens, h], np.float64))
    if parts:
        return out, o_soft, o_lin, n_lin
    return out


def hybrid_attn(inputs: dict, lay: Layout, readings: Readings = PRIMARY) -> np.ndarray:
    """Full layer forward.  Tensors (BNHD, numpy):
    q, k, v [B, T*P, H, d]; text_k, text_v [B, L, H, d];
    beta [B, T*P + L, H] (video tokens then text, R13); alpha [B, T, H];
    gate_logits [B, T*P, H, 2] (0 = softmax gate, 1 = linear gate).
    Returns O [B, T*P, H, d] in float64."""
    out = np.zeros(inputs["q"].shape, dtype=np.float64)
    tokens = np.arange(lay.video_tokens)
    for b in range(lay.batch):
        for h in range(lay.heads):
            out[b, :, h] = hybrid_attn_rows(inputs, lay, b, h, tokens, readings)
    return out


# ---------------------------------------------------------------------------
# Output projections (the step right after the layer)  [PD §三, figure 3]
# ---------------------------------------------------------------------------

def gated_branches_rows(inputs: dict, lay: Layout, b: int, tokens,
                        readings: Readings = PRIMARY) -> np.ndarray:
    """Gated branch outputs of the given video tokens of batch b, every head:
    [len(tokens), 2, H, d] with [:, 0, h] = sigmoid(l0) O_soft and
    [:, 1, h] = sigmoid(l1) RMSNorm(o_lin) [PD §三, figure 3]."""
    tokens = np.asarray(tokens)
    H, d = inputs["q"].shape[2], inputs["q"].shape[3]
    out = np.zeros((len(tokens), 2, H, d), dtype=np.float64)
    gates = np.asarray(inputs["gate_logits"], np.float64)
    for h in range(lay.heads):
        _, o_soft, _, n_lin = hybrid_attn_rows(inputs, lay, b, h, tokens, readings, parts=True)
        g = gates[b, tokens, h]
        out[:, 0, h] = _sigmoid(g[:, 0:1]) * o_soft
        out[:, 1, h] = _sigmoid(g[:, 1:2]) * n_lin
    return out


def gated_branches(inputs: dict, lay: Layout, readings: Readings = PRIMARY) -> np.ndarray:
    """The two gated branch outputs side by side, before their projections:
    X2[b, i, 0] = sigmoid(l0) O_soft and X2[b, i, 1] = sigmoid(l1) RMSNorm(o_lin),
    each [H, d], so a token's row is 2*H*d long, softmax branch first.  Their
    per-head sum is the layer output O [PD §三: each branch has its own gate
    and its own output projection, then both return to the residual]."""
    B, N, H, d = inputs["q"].shape
    x2 = np.zeros((B, N, 2, H, d), dtype=np.float64)
    tokens = np.arange(lay.video_tokens)
    for b in range(lay.batch):
        x2[b] = gated_branches_rows(inputs, lay, b, tokens, readings)
    return x2


def output_projection(x2, w_o) -> np.ndarray:
    """y = W_s (gated softmax branch) + W_l (gated linear branch), one product
    with the two weights side by side: w_o [d_model, 2*H*d] in (out, in)
    order, the first H*d input columns for the softmax branch, the rest for
    the linear branch.  x2 [B, N, 2, H, d] -> y [B, N, d_model]
    [PD §三; deepmagic blog 實測數據 (linear layers after the attention)]."""
    x2 = np.asarray(x2, np.float64)
    B, N = x2.shape[:2]
    return x2.reshape(B, N, -1) @ np.asarray(w_o, np.float64).T
