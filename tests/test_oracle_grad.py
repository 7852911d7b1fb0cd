"""Pins of the backward oracle (CPU).

``oracle.vdn_oracle_grad`` differentiates a torch float64 copy of the layer
forward.  It is pinned to things outside itself:

- its forward equals ``vdn_oracle.hybrid_attn`` (the pinned forward oracle);
- for every input, the directional derivative of ``vdn_oracle``'s own numpy
  forward, by central differences, equals <gradient, direction>;
- the gate-logit gradients equal their closed form
  (dO . branch) * sigmoid'(logit), built from ``vdn_oracle``'s branch outputs.
"""
import numpy as np
import pytest

from oracle import vdn_oracle as O
from oracle import vdn_oracle_grad as G
from video_diffusion_hybrid_block_amd import synth

from _helpers import custom, oracle_layout

CASES = [
    # far frames on both sides (chunks of 2, window 1), anchors, text
    dict(name="g_far", batch=1, heads=1, head_dim=4, frames=11, tokens_per_frame=3,
         text_tokens=2, dtype="f32", chunk_frames=2),
    # two heads, batch 2, no text (states start at zero), partial last chunk
    dict(name="g_notext", batch=2, heads=2, head_dim=3, frames=8, tokens_per_frame=2,
         text_tokens=0, dtype="f32", chunk_frames=3),
]


def _setup(case, **over):
    case = dict(case)
    af = case.pop("anchor_first", True)
    al = case.pop("anchor_last", True)
    w = custom(**case)
    inp = synth.make_inputs(w)
    inp = {k: np.asarray(a, np.float64) for k, a in inp.items()}
    lay = oracle_layout(w, anchor_first=af, anchor_last=al, **over)
    dO = np.random.default_rng(11).standard_normal(inp["q"].shape)
    return w, inp, lay, dO


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_forward_matches_the_forward_oracle(case):
    w, inp, lay, _ = _setup(case)
    np.testing.assert_allclose(G.hybrid_attn_forward(inp, lay), O.hybrid_attn(inp, lay),
                               rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_gradient_matches_central_differences_of_the_forward_oracle(case):
    w, inp, lay, dO = _setup(case)
    grads = G.hybrid_attn_grad(inp, lay, dO)
    rng = np.random.default_rng(3)

    def loss(x):
        return float(np.sum(dO * O.hybrid_attn(x, lay)))

    eps = 1e-6
    for key in G.GRAD_KEYS:
        if inp[key].size == 0:
            continue
        D = rng.standard_normal(inp[key].shape)
        xp = dict(inp); xp[key] = inp[key] + eps * D
        xm = dict(inp); xm[key] = inp[key] - eps * D
        fd = (loss(xp) - loss(xm)) / (2 * eps)
        an = float(np.sum(grads[key] * D))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (key, fd, an)


def test_gate_gradients_have_the_closed_form():
    w, inp, lay, dO = _setup(CASES[0])
    grads = G.hybrid_attn_grad(inp, lay, dO)
    toks = np.arange(lay.video_tokens)
    for b in range(lay.batch):
        for h in range(lay.heads):
            _, o_soft, _, n_lin = O.hybrid_attn_rows(inp, lay, b, h, toks, parts=True)
            g = inp["gate_logits"][b, :, h]
            s0, s1 = 1 / (1 + np.exp(-g[:, 0])), 1 / (1 + np.exp(-g[:, 1]))
            ref0 = np.sum(dO[b, :, h] * o_soft, axis=1) * s0 * (1 - s0)
            ref1 = np.sum(dO[b, :, h] * n_lin, axis=1) * s1 * (1 - s1)
            np.testing.assert_allclose(grads["gate_logits"][b, :, h, 0], ref0, rtol=1e-10, atol=1e-13)
            np.testing.assert_allclose(grads["gate_logits"][b, :, h, 1], ref1, rtol=1e-10, atol=1e-13)


def test_frames_outside_every_fold_get_no_state_gradient():
    """alpha and the video beta of frames no state folds (window frames of
    every chunk, anchors) do not reach the output: zero gradient."""
    w, inp, lay, dO = _setup(CASES[0])
    grads = G.hybrid_attn_grad(inp, lay, dO)
    folded = set()
    for t in range(lay.frames):
        folded |= set(O.far_forward(lay, t)) | set(O.far_backward(lay, t))
    P = lay.tokens_per_frame
    for f in range(lay.frames):
        if f not in folded:
            assert np.all(grads["alpha"][:, f] == 0)
            assert np.all(grads["beta"][:, f * P:(f + 1) * P] == 0)
        else:
            assert np.any(grads["alpha"][:, f] != 0)
