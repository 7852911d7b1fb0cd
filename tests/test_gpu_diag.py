"""Diagnostics of the library (not part of the method): with VDN_SYNC_DEBUG=1
and VDN_ROCTX=1 every stage synchronises, is checked and is bracketed by a
roctx range, and the results are unchanged bit for bit; no stage reports a
failure.  The environment is read on the library's first call, so the
diagnosed run is a child process; it compares against the parent's run of
the same layer and of the backward pass."""
import os
import subprocess
import sys

import pytest
import torch

from video_diffusion_hybrid_block_amd import binding as V
from video_diffusion_hybrid_block_amd import synth

from _helpers import custom, require_gpu, to_dev

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CASE = dict(name="diag", batch=1, heads=4, head_dim=128, frames=12, tokens_per_frame=96,
            text_tokens=32, dtype="bf16", seed=41, chunk_frames=3)

CHILD = r"""
import sys, torch
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
from video_diffusion_hybrid_block_amd import binding as V, synth
from _helpers import custom, to_dev
w = custom(**{case!r})
dev = to_dev(synth.make_inputs(w), w.dtype)
geo = dict(frames=w.frames, tokens_per_frame=w.tokens_per_frame, chunk_frames=w.chunk_frames,
           window_chunks=w.window_chunks)
args = (dev["q"], dev["k"], dev["v"], dev["text_k"], dev["text_v"], dev["beta"], dev["alpha"],
        dev["gate_logits"])
o = V.hybrid_attn(*args, **geo)
g = V.hybrid_attn_bwd(*args, torch.ones_like(o), **geo)
torch.cuda.synchronize()
assert V.last_failed_stage() is None, V.last_failed_stage()
torch.save({{"o": o.cpu(), "g": {{k: t.cpu() for k, t in g.items() if t is not None}}}}, sys.argv[1])
print("[child] done", flush=True)
"""


@pytest.mark.gpu
def test_sync_debug_and_roctx_leave_results_unchanged(tmp_path):
    require_gpu()
    w = custom(**CASE)
    dev = to_dev(synth.make_inputs(w), w.dtype)
    geo = dict(frames=w.frames, tokens_per_frame=w.tokens_per_frame, chunk_frames=w.chunk_frames,
               window_chunks=w.window_chunks)
    args = (dev["q"], dev["k"], dev["v"], dev["text_k"], dev["text_v"], dev["beta"],
            dev["alpha"], dev["gate_logits"])
    o = V.hybrid_attn(*args, **geo)
    g = V.hybrid_attn_bwd(*args, torch.ones_like(o), **geo)
    torch.cuda.synchronize()
    assert V.last_failed_stage() is None
    out = tmp_path / "diag.pt"
    env = dict(os.environ, VDN_SYNC_DEBUG="1", VDN_ROCTX="1")
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), case=CASE)
    print("\n[case] diagnosed child run", flush=True)
    r = subprocess.run([sys.executable, "-c", code, str(out)], env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    got = torch.load(out, weights_only=True)
    assert torch.equal(got["o"], o.cpu())
    for k, t in g.items():
        if t is not None:
            assert torch.equal(got["g"][k], t.cpu()), k
