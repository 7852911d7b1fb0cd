"""Gradients of the hybrid video attention layer (its backward pass), CPU,
float64.

TEST INFRASTRUCTURE ONLY.  Only ``tests/`` may import this module; the HIP
library and its Python binding never import it and share no code with it.

The backward pass is the gradient of the forward pass, so the oracle is that
gradient: the layer forward is written again with float64 CPU torch tensors,
step by step as in ``vdn_oracle`` (frame statistics, the joint per-frame
update by an SPD solve, the two folds from half of the text write over the
far frames, the summed read, RMSNorm, the sigmoid-gated merge, and one
softmax over the visible video keys and all text keys), and reverse-mode
automatic differentiation (``torch.autograd``, a library primitive) gives the
vector-Jacobian product with an upstream gradient dO for every input.  Which
frames are visible, far or anchors is ``vdn_oracle``'s integer geometry.
Only the primary readings of ``vdn_oracle`` are covered (the GPU implements
only those).

Sources as in ``vdn_oracle``: PaperDaily explainer "伯克利与Impossible视频生成"
§二–§四 (window, anchors, the two states and their half text write, gates and
RMSNorm, the joint per-frame update); deepmagic blog "生成比播放還快",
section 用兩條分支取代一條 (closed form S = (S̄ + B)(I + A)^-1).  The pages
describe no backward pass; training the new branch (PaperDaily §五, staged
alignment) needs this gradient.

Pins (``tests/test_oracle_grad.py``): the forward here equals
``vdn_oracle.hybrid_attn``; directional derivatives of ``vdn_oracle``'s own
forward by central differences match the gradient; the gate gradients match
their closed form.
"""
from __future__ import annotations

import numpy as np
import torch

from . import vdn_oracle as O

__all__ = ["layer_forward_bh", "hybrid_attn_forward", "hybrid_attn_grad",
           "hybrid_attn_grad_bh", "GRAD_KEYS"]

GRAD_KEYS = ("q", "k", "v", "text_k", "text_v", "beta", "alpha", "gate_logits")


def _stats(k_rows, v_rows, beta_rows):
    """A = sum_i beta_i k_i k_i^T, B = sum_i beta_i v_i k_i^T [DM 用兩條分支取代一條]."""
    A = (k_rows * beta_rows[:, None]).T @ k_rows
    B = (v_rows * beta_rows[:, None]).T @ k_rows
    return A, B


def _update(S_bar, A, B):
    """(S_bar + B)(I + A)^-1 by a solve with the SPD matrix I + A
    [DM 用兩條分支取代一條; PD §四]."""
    M = torch.eye(A.shape[0], dtype=A.dtype) + A
    return torch.linalg.solve(M, (S_bar + B).T).T


def layer_forward_bh(q, k, v, tk, tv, beta, alpha, gates, lay: O.Layout):
    """Layer output of one (batch, head) as a torch float64 tensor [N, d].
    q, k, v [N, d]; tk, tv [L, d]; beta [N + L]; alpha [T]; gates [N, 2]."""
    P, T, L = lay.tokens_per_frame, lay.frames, lay.text_tokens
    N = T * P
    d_v, d_k = v.shape[1], k.shape[1]

    def rows(f):
        return slice(f * P, (f + 1) * P)

    # half of the text write starts both states [PD §三]
    if L > 0:
        Ax, Bx = _stats(tk, tv, beta[N:N + L])
        S0 = 0.5 * _update(torch.zeros(d_v, d_k, dtype=q.dtype), Ax, Bx)
    else:
        S0 = torch.zeros(d_v, d_k, dtype=q.dtype)
    stats = {}

    def stat(f):
        if f not in stats:
            stats[f] = _stats(k[rows(f)], v[rows(f)], beta[rows(f)])
        return stats[f]

    def fold(frames):
        S = S0
        for f in frames:
            A, B = stat(f)
            S = _update(alpha[f] * S, A, B)
        return S

    out = []
    for t in range(T):
        vis = O.visible_frames(lay, t)
        K = torch.cat([k[rows(f)] for f in vis] + ([tk] if L > 0 else []))
        V = torch.cat([v[rows(f)] for f in vis] + ([tv] if L > 0 else []))
        Q = q[rows(t)]
        o_soft = torch.softmax((Q @ K.T) * lay.scale, dim=1) @ V
        R = fold(O.far_forward(lay, t)) + fold(O.far_backward(lay, t))
        o_lin = Q @ R.T
        n_lin = o_lin / torch.sqrt(torch.mean(o_lin * o_lin, dim=1, keepdim=True) + lay.rms_eps)
        g = gates[rows(t)]
        out.append(torch.sigmoid(g[:, 0:1]) * o_soft + torch.sigmoid(g[:, 1:2]) * n_lin)
    return torch.cat(out)


def _bh_tensors(inputs: dict, lay: O.Layout, b: int, h: int, requires_grad: bool):
    N, L = lay.video_tokens, lay.text_tokens
    d = inputs["q"].shape[-1]

    def t(a):
        return torch.tensor(np.asarray(a, np.float64), requires_grad=requires_grad)

    tk = inputs["text_k"][b, :, h] if L > 0 else np.zeros((0, d))
    tv = inputs["text_v"][b, :, h] if L > 0 else np.zeros((0, d))
    return dict(q=t(inputs["q"][b, :, h]), k=t(inputs["k"][b, :, h]), v=t(inputs["v"][b, :, h]),
                text_k=t(tk), text_v=t(tv), beta=t(inputs["beta"][b, :N + L, h]),
                alpha=t(inputs["alpha"][b, :, h]), gate_logits=t(inputs["gate_logits"][b, :, h]))


def _call(x: dict, lay: O.Layout):
    return layer_forward_bh(x["q"], x["k"], x["v"], x["text_k"], x["text_v"], x["beta"],
                            x["alpha"], x["gate_logits"], lay)


def hybrid_attn_forward(inputs: dict, lay: O.Layout) -> np.ndarray:
    """The layer output O [B, N, H, d] from this module's torch forward."""
    out = np.zeros(inputs["q"].shape, np.float64)
    with torch.no_grad():
        for b in range(lay.batch):
            for h in range(lay.heads):
                out[b, :, h] = _call(_bh_tensors(inputs, lay, b, h, False), lay).numpy()
    return out


def hybrid_attn_grad_bh(inputs: dict, lay: O.Layout, dO, b: int, h: int) -> dict:
    """Gradients of sum(dO * O) restricted to one (batch, head): heads and
    batch entries do not interact, so this is that slice of the full
    gradient.  Arrays shaped like the inputs' (b, :, h) slices."""
    x = _bh_tensors(inputs, lay, b, h, True)
    out = _call(x, lay)
    out.backward(torch.tensor(np.asarray(dO[b, :, h], np.float64)))
    res = {}
    for key in GRAD_KEYS:
        t = x[key]
        # an input the output does not depend on has no gradient
        res[key] = np.zeros(tuple(t.shape)) if t.grad is None else t.grad.numpy()
    return res


def hybrid_attn_grad(inputs: dict, lay: O.Layout, dO) -> dict:
    """Gradient of sum(dO * O) with respect to each input of the layer, as
    float64 arrays shaped like the inputs (``GRAD_KEYS``).  beta's gradient
    covers video then text tokens like beta itself."""
    dO = np.asarray(dO, np.float64)
    N, L = lay.video_tokens, lay.text_tokens
    grads = {key: np.zeros(np.shape(inputs[key]), np.float64) for key in GRAD_KEYS
             if inputs.get(key) is not None}
    for b in range(lay.batch):
        for h in range(lay.heads):
            r = hybrid_attn_grad_bh(inputs, lay, dO, b, h)
            grads["q"][b, :, h] = r["q"]
            grads["k"][b, :, h] = r["k"]
            grads["v"][b, :, h] = r["v"]
            if L > 0:
                grads["text_k"][b, :, h] = r["text_k"]
                grads["text_v"][b, :, h] = r["text_v"]
            grads["beta"][b, :N + L, h] = r["beta"]
            grads["alpha"][b, :, h] = r["alpha"]
            grads["gate_logits"][b, :, h] = r["gate_logits"]
    return grads
