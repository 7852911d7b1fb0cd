"""GPU parity of the layer on seeded random layouts against the CPU oracle.

A fixed-seed draw of small layouts across the whole layout space the C ABI
accepts: head size (16, 32, 64, 128), dtype (bf16, fp32), frames (1-14),
tokens per frame (1-200, multiples of 8 or not, so both softmax paths run),
text tokens (0-40), chunk length (1-5), window (0-3 chunks), either anchor
on or off, batch and heads.  Each layout is small enough for the fp64 oracle
to finish in about a second; the bounds are the layer's (1e-4 fp32, 2e-2
bf16 relative Frobenius error).
"""
import numpy as np
import pytest

from oracle import vdn_oracle as O
from video_diffusion_hybrid_block_amd import binding as V
from video_diffusion_hybrid_block_amd import synth

from _helpers import TOL, custom, oracle_layout, rel_err, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _draw(n=32, seed=20261204):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        d = int(rng.choice([16, 32, 64, 128], p=[0.1, 0.3, 0.3, 0.3]))
        P = int(rng.choice([int(rng.integers(1, 9)) * 8, int(rng.integers(1, 201))]))
        frames = int(rng.integers(1, 15))
        while frames * P > 1600:
            frames = max(1, frames // 2)
        cases.append(dict(
            name=f"rand{i:02d}", batch=int(rng.integers(1, 3)), heads=int(rng.integers(1, 3)),
            head_dim=d, frames=frames, tokens_per_frame=P,
            text_tokens=int(rng.choice([0, 8, 16, int(rng.integers(1, 41))])),
            dtype="bf16" if i % 2 == 0 else "f32", seed=500 + i,
            chunk_frames=int(rng.integers(1, 6)), window_chunks=int(rng.integers(0, 4)),
            anchor_first=bool(rng.random() < 0.8), anchor_last=bool(rng.random() < 0.8)))
    return cases


CASES = _draw()


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_layer_random_layout(case):
    require_gpu()
    case = dict(case)
    af, al = case.pop("anchor_first"), case.pop("anchor_last")
    w = custom(**case)
    print(f"\n[case] {case}", flush=True)
    inp = synth.make_inputs(w)
    ref = O.hybrid_attn(inp, oracle_layout(w, anchor_first=af, anchor_last=al))
    dev = to_dev(inp, w.dtype)
    L = w.text_tokens
    out = V.hybrid_attn(dev["q"], dev["k"], dev["v"], dev["text_k"] if L else None,
                        dev["text_v"] if L else None, dev["beta"], dev["alpha"],
                        dev["gate_logits"], frames=w.frames, tokens_per_frame=w.tokens_per_frame,
                        chunk_frames=w.chunk_frames, window_chunks=w.window_chunks,
                        anchor_first=af, anchor_last=al)
    out = out.float().cpu().numpy()
    err = rel_err(out, ref)
    print(f"{case['name']}: rel err {err:.3e}", flush=True)
    assert np.isfinite(out).all()
    assert err <= TOL[w.dtype]
