"""GPU parity of the backward pass (vdn_hybrid_attn_bwd, through the C ABI)
against the backward oracle (oracle.vdn_oracle_grad) on the same seeded
inputs and upstream gradient.

Metric: relative Frobenius error per gradient tensor.  Bound 2e-2 (the bf16
layer tolerance): the gradients run through the same bf16 roundings as the
forward (P, the scan's three-pass products) plus bf16 dO_s and dS operands.
"""
import numpy as np
import pytest
import torch

from oracle import vdn_oracle as O
from oracle import vdn_oracle_grad as G
from video_diffusion_hybrid_block_amd import binding as V
from video_diffusion_hybrid_block_amd import synth

from _helpers import custom, oracle_layout, rel_err, require_gpu, to_dev

pytestmark = pytest.mark.gpu

TOL = 2e-2
# Saved-residual backward against the recomputing one: the two compute D =
# dO_s . O_s in different summation orders (about 1e-7 relative), and dS is
# rounded to bf16 before the dq and dk products, so that difference flips
# the rounding of an occasional dS element; one flip moves dq or dk by about
# 1e-5 of its norm at these sizes.  A wrong residual moves them by far more.
TRAIN_TOL = 1e-4
# The training forward forms its softmax scores exactly in fp32 (its
# log-sum-exp drives the backward); the layer forms them from q * scale *
# log2(e) rounded to bf16.  On unit keys against N(0, 1) queries the two
# differ by ~1e-4 before the outputs are rounded to bf16, which then flips
# the rounding of a few per cent of the elements by one bf16 step (2^-8
# relative): up to ~2e-3 of the norm.  Both also meet the oracle bound.
FWD_TOL = 5e-3


def _out_close(o, o_ref):
    d = float(torch.linalg.vector_norm((o.double() - o_ref.double()))
              / torch.linalg.vector_norm(o_ref.double()))
    print(f"training forward vs layer output: {d:.2e}", flush=True)
    return d <= FWD_TOL

CASES = [
    # far frames on both sides, anchors, text; two 256-query tiles per frame
    dict(name="bwd_d64", batch=1, heads=2, head_dim=64, frames=12, tokens_per_frame=104,
         text_tokens=16, dtype="bf16", chunk_frames=3),
    # d = 128, batch 2, 128-key tiles with a ragged tail, text
    dict(name="bwd_d128_b2", batch=2, heads=2, head_dim=128, frames=7, tokens_per_frame=136,
         text_tokens=24, dtype="bf16", chunk_frames=2),
    # d = 32, no text (states start at zero), partial last chunk
    dict(name="bwd_d32_notext", batch=1, heads=3, head_dim=32, frames=10, tokens_per_frame=40,
         text_tokens=0, dtype="bf16", chunk_frames=3),
    # the linear branch gated off (sigmoid(-30)): dq, dk, dv are the softmax
    # backward alone
    dict(name="bwd_softmax_only", batch=1, heads=2, head_dim=128, frames=9, tokens_per_frame=72,
         text_tokens=16, dtype="bf16", chunk_frames=2, gates=(4.0, -30.0)),
    # the softmax branch gated off: the linear branch's gradients alone
    dict(name="bwd_linear_only", batch=1, heads=2, head_dim=64, frames=13, tokens_per_frame=48,
         text_tokens=8, dtype="bf16", chunk_frames=2, gates=(-30.0, 4.0)),
    # one frame: every query is an anchor query, no far frames, no text
    dict(name="bwd_one_frame", batch=1, heads=2, head_dim=64, frames=1, tokens_per_frame=200,
         text_tokens=0, dtype="bf16"),
    # window wider than the video: dense softmax, linear read = text write
    dict(name="bwd_dense_window", batch=1, heads=1, head_dim=128, frames=9, tokens_per_frame=48,
         text_tokens=16, dtype="bf16", chunk_frames=2, window_chunks=5),
    dict(name="bwd_no_anchors", batch=1, heads=2, head_dim=64, frames=12, tokens_per_frame=40,
         text_tokens=8, dtype="bf16", chunk_frames=3, anchor_first=False, anchor_last=False),
    dict(name="bwd_last_anchor_only", batch=1, heads=1, head_dim=32, frames=14, tokens_per_frame=24,
         text_tokens=8, dtype="bf16", chunk_frames=2, anchor_first=False),
]


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_backward_matches_oracle(case):
    require_gpu()
    case = dict(case)
    af = case.pop("anchor_first", True)
    al = case.pop("anchor_last", True)
    gates = case.pop("gates", None)
    w = custom(**case)
    _announce(f"backward {case['name']}")
    inp = synth.make_inputs(w)
    if gates is not None:
        inp["gate_logits"][..., 0] += gates[0]
        inp["gate_logits"][..., 1] += gates[1]
    lay = oracle_layout(w, anchor_first=af, anchor_last=al)
    dO = synth.round_bf16(np.random.default_rng(w.seed + 7).standard_normal(inp["q"].shape))
    ref = G.hybrid_attn_grad({k_: np.asarray(a, np.float64) for k_, a in inp.items()}, lay, dO)
    dev = to_dev(inp, w.dtype)
    L = w.text_tokens
    got = V.hybrid_attn_bwd(dev["q"], dev["k"], dev["v"], dev["text_k"] if L else None,
                            dev["text_v"] if L else None, dev["beta"], dev["alpha"],
                            dev["gate_logits"], torch.from_numpy(dO).to(torch.bfloat16).cuda(),
                            frames=w.frames, tokens_per_frame=w.tokens_per_frame,
                            chunk_frames=w.chunk_frames, window_chunks=w.window_chunks,
                            anchor_first=af, anchor_last=al)
    torch.cuda.synchronize()
    errs = {}
    for key in G.GRAD_KEYS:
        if got.get(key) is None:
            continue
        g = got[key].cpu().numpy()
        assert np.isfinite(g).all(), key
        if np.linalg.norm(ref[key]) < 1e-30:
            # no gradient at all (e.g. alpha and beta with no folded frame)
            errs[key] = float(np.abs(g).max())
            continue
        errs[key] = rel_err(g, ref[key])
    print(case["name"], " ".join(f"{k_} {e:.2e}" for k_, e in errs.items()), flush=True)
    bad = {k_: e for k_, e in errs.items() if not e <= TOL}
    assert not bad, bad


@pytest.mark.timeout(900)
def test_backward_768p_one_head_in_full():
    """The 768p layer (B=1, H=24, d=128, 60 x 1008 tokens, 512 text tokens)
    in the launch configuration bench.py times: heads do not interact, so
    head 0's slice of every gradient is compared in full with the oracle's
    gradient of that head."""
    require_gpu()
    from _helpers import workload
    w = workload("768p")
    _announce("backward 768p head 0")
    inp = synth.make_inputs(w)
    lay = oracle_layout(w)
    dO = synth.round_bf16(np.random.default_rng(w.seed + 7).standard_normal(
        inp["q"].shape).astype(np.float32))
    dev = to_dev(inp, w.dtype)
    got = V.hybrid_attn_bwd(dev["q"], dev["k"], dev["v"], dev["text_k"], dev["text_v"],
                            dev["beta"], dev["alpha"], dev["gate_logits"],
                            torch.from_numpy(dO).to(torch.bfloat16).cuda(), frames=w.frames,
                            tokens_per_frame=w.tokens_per_frame, chunk_frames=w.chunk_frames,
                            window_chunks=w.window_chunks)
    torch.cuda.synchronize()
    got = {k_: (None if t is None else t[0, :, 0].cpu().numpy()) for k_, t in got.items()}
    del dev
    torch.cuda.empty_cache()
    print("[case] oracle gradient of head 0 (tens of seconds)", flush=True)
    ref = G.hybrid_attn_grad_bh(inp, lay, dO, 0, 0)
    errs = {k_: rel_err(got[k_], ref[k_]) for k_ in G.GRAD_KEYS}
    print("768p head 0", " ".join(f"{k_} {e:.2e}" for k_, e in errs.items()), flush=True)
    bad = {k_: e for k_, e in errs.items() if not e <= TOL}
    assert not bad, bad


def _grads_close(got, ref):
    errs = {}
    for key in G.GRAD_KEYS:
        if ref.get(key) is None:
            continue
        a, b = got[key].double(), ref[key].double()
        assert torch.isfinite(a).all(), key
        nb = torch.linalg.vector_norm(b)
        errs[key] = float(torch.linalg.vector_norm(a - b) / nb) if nb > 0 else \
            float(a.abs().max())
    return errs


TRAIN_CASES = [CASES[0], CASES[1], CASES[2], CASES[4], CASES[5]]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", TRAIN_CASES, ids=[c["name"] for c in TRAIN_CASES])
def test_training_pair_matches_recompute_and_oracle(case):
    """vdn_hybrid_attn_fwd_train + vdn_hybrid_attn_bwd_saved: the output is
    vdn_hybrid_attn_fwd's up to its score rounding (FWD_TOL) and meets the
    oracle bound; the gradients equal
    vdn_hybrid_attn_bwd's up to the summation order of the merge backward's
    dot products (TRAIN_TOL) and meet the oracle bound.  Layouts: d = 64
    with text, d = 128 with batch 2 and a ragged tile, d = 32 without text,
    the softmax branch gated off, one frame."""
    require_gpu()
    case = dict(case)
    af = case.pop("anchor_first", True)
    al = case.pop("anchor_last", True)
    gates = case.pop("gates", None)
    w = custom(**case)
    _announce(f"training pair {case['name']}")
    inp = synth.make_inputs(w)
    if gates is not None:
        inp["gate_logits"][..., 0] += gates[0]
        inp["gate_logits"][..., 1] += gates[1]
    lay = oracle_layout(w, anchor_first=af, anchor_last=al)
    dO = synth.round_bf16(np.random.default_rng(w.seed + 7).standard_normal(inp["q"].shape))
    dev = to_dev(inp, w.dtype)
    L = w.text_tokens
    args = (dev["q"], dev["k"], dev["v"], dev["text_k"] if L else None,
            dev["text_v"] if L else None, dev["beta"], dev["alpha"], dev["gate_logits"])
    geo = dict(frames=w.frames, tokens_per_frame=w.tokens_per_frame,
               chunk_frames=w.chunk_frames, window_chunks=w.window_chunks,
               anchor_first=af, anchor_last=al)
    dOd = torch.from_numpy(dO).to(torch.bfloat16).cuda()
    o_ref = V.hybrid_attn(*args, **geo)
    o, saved = V.hybrid_attn_fwd_train(*args, **geo)
    g_saved = V.hybrid_attn_bwd_saved(*args, dOd, saved, **geo)
    g_re = V.hybrid_attn_bwd(*args, dOd, **geo)
    torch.cuda.synchronize()
    assert _out_close(o, o_ref)
    oe = rel_err(o.float().cpu().numpy(), O.hybrid_attn(inp, lay))
    print(case["name"], f"training forward vs oracle {oe:.2e}", flush=True)
    assert oe <= TOL
    errs = _grads_close(g_saved, g_re)
    print(case["name"], "saved vs recompute", " ".join(f"{k_} {e:.1e}" for k_, e in errs.items()),
          flush=True)
    bad = {k_: e for k_, e in errs.items() if not e <= TRAIN_TOL}
    assert not bad, bad
    ref = G.hybrid_attn_grad({k_: np.asarray(a, np.float64) for k_, a in inp.items()}, lay, dO)
    oerr = {}
    for key in G.GRAD_KEYS:
        if g_saved.get(key) is None:
            continue
        g = g_saved[key].cpu().numpy()
        oerr[key] = (float(np.abs(g).max()) if np.linalg.norm(ref[key]) < 1e-30
                     else rel_err(g, ref[key]))
    bad = {k_: e for k_, e in oerr.items() if not e <= TOL}
    assert not bad, bad


@pytest.mark.timeout(600)
def test_training_pair_768p_matches_recompute():
    """The 768p layer in the launch configuration bench.py times: every
    gradient of the saved-residual backward against the recomputing backward
    over all heads (TRAIN_TOL), and the output against the layer's
    (FWD_TOL)."""
    require_gpu()
    from _helpers import workload
    w = workload("768p")
    _announce("training pair 768p")
    inp = synth.make_inputs(w)
    dO = synth.round_bf16(np.random.default_rng(w.seed + 7).standard_normal(
        inp["q"].shape).astype(np.float32))
    dev = to_dev(inp, w.dtype)
    args = (dev["q"], dev["k"], dev["v"], dev["text_k"], dev["text_v"], dev["beta"],
            dev["alpha"], dev["gate_logits"])
    geo = dict(frames=w.frames, tokens_per_frame=w.tokens_per_frame,
               chunk_frames=w.chunk_frames, window_chunks=w.window_chunks)
    dOd = torch.from_numpy(dO).to(torch.bfloat16).cuda()
    o_ref = V.hybrid_attn(*args, **geo)
    o, saved = V.hybrid_attn_fwd_train(*args, **geo)
    g_saved = V.hybrid_attn_bwd_saved(*args, dOd, saved, **geo)
    del saved
    g_re = V.hybrid_attn_bwd(*args, dOd, **geo)
    torch.cuda.synchronize()
    assert _out_close(o, o_ref)
    errs = _grads_close(g_saved, g_re)
    print("768p saved vs recompute", " ".join(f"{k_} {e:.1e}" for k_, e in errs.items()),
          flush=True)
    bad = {k_: e for k_, e in errs.items() if not e <= TRAIN_TOL}
    assert not bad, bad


@pytest.mark.timeout(600)
def test_training_pair_reuses_one_saved_buffer():
    """One saved buffer serves consecutive training steps: a step on new
    inputs (other q, v and gate logits) after a step on the first ones gives
    bit for bit what a fresh buffer gives, so nothing of the first step
    leaks into the second."""
    require_gpu()
    case = dict(CASES[0])
    case.pop("anchor_first", None)
    case.pop("anchor_last", None)
    w = custom(**case)
    _announce("training pair, saved buffer reused")
    inp = synth.make_inputs(w)
    dO = synth.round_bf16(np.random.default_rng(w.seed + 7).standard_normal(inp["q"].shape))
    dev = to_dev(inp, w.dtype)
    dev2 = dict(dev)
    dev2["q"] = dev["q"].flip(1).contiguous()
    dev2["v"] = dev["v"].flip(1).contiguous()
    dev2["gate_logits"] = -dev["gate_logits"]
    geo = dict(frames=w.frames, tokens_per_frame=w.tokens_per_frame,
               chunk_frames=w.chunk_frames, window_chunks=w.window_chunks)
    dOd = torch.from_numpy(dO).to(torch.bfloat16).cuda()

    def step(d, saved):
        args = (d["q"], d["k"], d["v"], d["text_k"], d["text_v"], d["beta"], d["alpha"],
                d["gate_logits"])
        o, saved = V.hybrid_attn_fwd_train(*args, **geo, saved=saved)
        g = V.hybrid_attn_bwd_saved(*args, dOd, saved, **geo)
        return o, g, saved

    _, _, saved = step(dev, None)
    o_reused, g_reused, _ = step(dev2, saved)
    o_fresh, g_fresh, _ = step(dev2, None)
    torch.cuda.synchronize()
    assert torch.equal(o_reused.view(torch.int16), o_fresh.view(torch.int16))
    for key in G.GRAD_KEYS:
        if g_fresh.get(key) is None:
            continue
        assert torch.equal(g_reused[key], g_fresh[key]), key
