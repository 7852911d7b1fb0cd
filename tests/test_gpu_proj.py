"""GPU parity of the separate output projections (through the C ABI).

Stages checked against the oracle on the same seeded inputs:
- the projection product alone (vdn_out_proj) against oracle.output_projection
  on bf16 operands, ragged M and N, K from one 64-step to the 768p 6144;
- the gated branches kept apart (vdn_softmax_branches_fwd) against
  oracle.gated_branches, each branch on its own;
- the layer with its projections (vdn_hybrid_attn_proj_fwd) against
  oracle.output_projection(oracle.gated_branches(...)), small shapes in full
  and the 768p shape on sampled tokens;
- the FP8 (MXFP8) forms: quantization bit-exact against oracle.mx_fp8, the
  FP8 product against the exact product of the quantized operands, the
  branches quantized inside the softmax kernel against the exact branches
  and their MX quantization, and the layer with FP8 projections.

Metric: relative Frobenius error.  Bounds: the product rounds each output to
bf16 (relative 2^-9) after an fp32 sum, so 4e-3; the branch and layer outputs
carry the softmax's bf16 P and the bf16 rounding of x2 on top, so 1e-2 per
branch and 2e-2 on y (the layer tolerance).
"""
import numpy as np
import pytest
import torch

from oracle import vdn_oracle as O
from video_diffusion_hybrid_block_amd import binding as V
from video_diffusion_hybrid_block_amd import synth

from _helpers import (TOL, custom, oracle_chunk_reads, oracle_layout, rel_err, require_gpu,
                      to_dev, workload)

pytestmark = pytest.mark.gpu

GEMM_TOL = 4e-3


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).cuda()


GEMM_SHAPES = [
    (1, 64, 8),          # one token, one k step, one 8-wide output group
    (300, 192, 264),     # ragged in M and N, three k steps
    (513, 640, 520),     # two full M tiles + a 1-row tail; N tail of 8
    (2048, 6144, 512),   # the 768p K, eight M tiles
]


@pytest.mark.parametrize("M,K,N", GEMM_SHAPES, ids=[f"{m}x{k}x{n}" for m, k, n in GEMM_SHAPES])
def test_out_proj_product(M, K, N):
    require_gpu()
    _announce(f"out_proj M={M} K={K} N={N}")
    x, w = synth.make_gemm_operands(M, K, N, seed=M + K + N)
    ref = O.output_projection(x.reshape(1, M, K), w)[0]
    y = V.out_proj(_bf16(x), _bf16(w))
    torch.cuda.synchronize()
    got = y.float().cpu().numpy()
    err = rel_err(got, ref)
    print(f"out_proj {M}x{K}x{N}: rel err {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= GEMM_TOL


def test_out_proj_768p_sampled_rows():
    """The 768p product (M = 60480 tokens, K = 2*24*128, N = 3072) in the
    launch configuration the layer uses; rows spanning the first, middle and
    ragged last M tile are checked against the oracle."""
    require_gpu()
    M, K, N = 60480, 6144, 3072
    _announce(f"out_proj 768p M={M} K={K} N={N}")
    x, w = synth.make_gemm_operands(M, K, N, seed=4242)
    y = V.out_proj(_bf16(x), _bf16(w))
    torch.cuda.synchronize()
    rows = np.array([0, 1, 31, 32, 255, 256, 30000, 30257, M - 193, M - 65, M - 2, M - 1])
    ref = O.output_projection(x[rows].reshape(1, len(rows), K), w)[0]
    got = y[torch.from_numpy(rows).cuda()].float().cpu().numpy()
    err = rel_err(got, ref)
    print(f"out_proj 768p sampled rows: rel err {err:.3e}")
    assert err <= GEMM_TOL


def test_out_proj_rejects_bad_shapes():
    require_gpu()
    x = torch.zeros((4, 96), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((8, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(V.VdnError) as e:
        V.out_proj(x, w)                      # K not a multiple of 64
    assert e.value.status == 3
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((12, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(V.VdnError) as e:
        V.out_proj(x, w)                      # N not a multiple of 8
    assert e.value.status == 3


BRANCH_CASES = [
    dict(name="branches_d64", batch=1, heads=8, head_dim=64, frames=30, tokens_per_frame=112,
         text_tokens=64, dtype="bf16", chunk_frames=5),
    dict(name="branches_d128", batch=1, heads=2, head_dim=128, frames=7, tokens_per_frame=600,
         text_tokens=24, dtype="bf16", chunk_frames=3),
    dict(name="branches_d32_b2", batch=2, heads=3, head_dim=32, frames=6, tokens_per_frame=40,
         text_tokens=0, dtype="bf16", chunk_frames=2),
]


@pytest.mark.parametrize("case", BRANCH_CASES, ids=[c["name"] for c in BRANCH_CASES])
def test_stage_softmax_branches(case):
    require_gpu()
    w = custom(**case)
    _announce(f"branches {case['name']}")
    inp = synth.make_inputs(w)
    lay = oracle_layout(w)
    ref = O.gated_branches(inp, lay)
    R = oracle_chunk_reads(inp, lay, w)
    dev = to_dev(inp, w.dtype)
    L = w.text_tokens
    x2 = V.softmax_branches_fwd(dev["q"], dev["k"], dev["v"], dev["text_k"] if L else None,
                                dev["text_v"] if L else None, torch.from_numpy(R).cuda(),
                                dev["gate_logits"], frames=w.frames,
                                tokens_per_frame=w.tokens_per_frame, chunk_frames=w.chunk_frames,
                                window_chunks=w.window_chunks)
    torch.cuda.synchronize()
    got = x2.float().cpu().numpy()
    e_s = rel_err(got[:, :, 0], ref[:, :, 0])
    e_l = rel_err(got[:, :, 1], ref[:, :, 1])
    print(f"{case['name']}: softmax branch rel err {e_s:.3e}, linear branch {e_l:.3e}")
    assert np.isfinite(got).all()
    assert e_s <= 1e-2 and e_l <= 1e-2


PROJ_LAYER_CASES = [
    dict(name="proj_layer_d64", batch=1, heads=4, head_dim=64, frames=12, tokens_per_frame=104,
         text_tokens=16, dtype="bf16", chunk_frames=3, d_model=264),
    dict(name="proj_layer_d128_b2", batch=2, heads=2, head_dim=128, frames=5, tokens_per_frame=200,
         text_tokens=8, dtype="bf16", chunk_frames=2, d_model=256),
    dict(name="proj_layer_d32", batch=1, heads=3, head_dim=32, frames=9, tokens_per_frame=24,
         text_tokens=0, dtype="bf16", chunk_frames=3, d_model=8),
]


def _run_proj_layer(w, inp, w_o):
    dev = to_dev(inp, w.dtype)
    L = w.text_tokens
    y = V.hybrid_attn_proj(dev["q"], dev["k"], dev["v"], dev["text_k"] if L else None,
                           dev["text_v"] if L else None, dev["beta"], dev["alpha"],
                           dev["gate_logits"], _bf16(w_o), frames=w.frames,
                           tokens_per_frame=w.tokens_per_frame, chunk_frames=w.chunk_frames,
                           window_chunks=w.window_chunks)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("case", PROJ_LAYER_CASES, ids=[c["name"] for c in PROJ_LAYER_CASES])
def test_layer_with_projections(case):
    require_gpu()
    case = dict(case)
    dm = case.pop("d_model")
    w = custom(**case)
    _announce(f"layer+proj {case['name']} d_model={dm}")
    inp = synth.make_inputs(w)
    lay = oracle_layout(w)
    w_o = synth.make_proj_weight(dm, w.heads, w.head_dim, seed=w.seed + 1)
    ref = O.output_projection(O.gated_branches(inp, lay), w_o)
    got = _run_proj_layer(w, inp, w_o).float().cpu().numpy()
    err = rel_err(got, ref)
    print(f"{case['name']}: layer+proj rel err {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= TOL["bf16"]


@pytest.mark.timeout(900)
def test_layer_with_projections_768p_sampled():
    """768p (H = 24, d = 128, d_model = H*d = 3072): y of sampled tokens
    (anchor, window-edge and interior frames; tile starts and the ragged end of
    a frame) against the oracle's branches of those tokens, all heads."""
    require_gpu()
    w = workload("768p")
    _announce("layer+proj 768p sampled")
    inp = synth.make_inputs(w)
    lay = oracle_layout(w)
    dm = w.heads * w.head_dim
    w_o = synth.make_proj_weight(dm, w.heads, w.head_dim, seed=w.seed + 1)
    y = _run_proj_layer(w, inp, w_o)
    P, T = w.tokens_per_frame, w.frames
    tok = np.array([f * P + x for f in (0, 1, 5, T // 2, T - 6, T - 1)
                    for x in (0, 255, 256, P - 1)])
    x2 = O.gated_branches_rows(inp, lay, 0, tok)
    ref = O.output_projection(x2[None], w_o)[0]
    got = y[0, torch.from_numpy(tok).cuda()].float().cpu().numpy()
    err = rel_err(got, ref)
    print(f"768p layer+proj sampled ({len(tok)} tokens): rel err {err:.3e}")
    assert err <= TOL["bf16"]


# ---------------------------------------------------------------------------
# FP8 (MXFP8) projections
# ---------------------------------------------------------------------------
from oracle import mx_fp8 as MX  # noqa: E402


def _codes_to_float(q):
    return q.view(torch.float8_e4m3fn).to(torch.float64).cpu().numpy()


def test_mxfp8_quantize_matches_oracle_exactly():
    """Codes and scales equal the oracle's (same bf16 inputs, so the same
    rounding decisions): blocks spanning many binades, zero blocks, values
    that clamp at the top and underflow at the bottom of a block."""
    require_gpu()
    _announce("mxfp8 quantize")
    rng = np.random.default_rng(11)
    M, K = 257, 320
    x = rng.standard_normal((M, K)) * np.exp2(rng.integers(-30, 30, (M, K // 32)).repeat(32, axis=1))
    x[:, 64:96] = 0.0                                 # zero blocks
    x[5, :32] = np.exp2(rng.integers(-20, 1, 32))     # one block over 20 binades
    x[6, :32] = 1.9375 * 2.0 ** 8                     # rounds up to the block's clamp
    xb = synth.round_bf16(x.astype(np.float32))
    q, s = V.mxfp8_quantize(_bf16(xb))
    torch.cuda.synchronize()
    P, X = MX.mx_quantize(xb.astype(np.float64))
    np.testing.assert_array_equal(s.cpu().numpy().astype(np.int64) - 127, X)
    np.testing.assert_array_equal(_codes_to_float(q), P)


def _e4m3_half_step(v, X):
    """Half the E4M3 spacing at |v| in a block with exponent X (scaled units
    u = v / 2^X: 3 mantissa bits, no binade below 2^-6), plus what the clamp
    at 448 removes; in the units of v."""
    u = np.abs(v) / np.exp2(X)
    with np.errstate(divide="ignore"):
        e = np.maximum(np.floor(np.log2(np.where(u > 0, u, 1.0))), -6.0)
    return (0.5 * np.exp2(e - 3) + np.maximum(u - 448.0, 0.0)) * np.exp2(X)


@pytest.mark.parametrize("case", BRANCH_CASES, ids=[c["name"] for c in BRANCH_CASES])
def test_stage_softmax_branches_mxfp8(case):
    """The gated branches written as MXFP8 by the softmax kernel
    (vdn_softmax_branches_mxfp8_fwd) against the oracle's exact branches and
    their MX quantization.  The kernel quantizes its own fp32 values, so where
    a value or a block maximum sits next to a rounding boundary either side
    of it is a valid result; what is checked:
    - block exponents equal the oracle's, or differ by one (a block maximum
      next to a power of two), for at least 99 % of blocks equal;
    - every element lies within half an E4M3 step (at the kernel's exponent)
      of the exact branch value, plus 1e-2 of its block maximum for the
      branch's own bf16 arithmetic (the bound of the bf16 branch test);
    - per branch, the dequantized values are as close to the exact ones as
      the oracle's own quantization: rel err <= 1.1 x the oracle's + 2e-3."""
    require_gpu()
    w = custom(**case)
    _announce(f"branches mxfp8 {case['name']}")
    inp = synth.make_inputs(w)
    lay = oracle_layout(w)
    B, N, H, d = w.batch, w.video_tokens, w.heads, w.head_dim
    ref = O.gated_branches(inp, lay).reshape(B * N, 2 * H * d)
    P_ref, X_ref = MX.mx_quantize(ref)
    R = oracle_chunk_reads(inp, lay, w)
    dev = to_dev(inp, w.dtype)
    L = w.text_tokens
    codes, scales = V.softmax_branches_mxfp8(dev["q"], dev["k"], dev["v"],
                                             dev["text_k"] if L else None,
                                             dev["text_v"] if L else None,
                                             torch.from_numpy(R).cuda(), dev["gate_logits"],
                                             frames=w.frames, tokens_per_frame=w.tokens_per_frame,
                                             chunk_frames=w.chunk_frames,
                                             window_chunks=w.window_chunks)
    torch.cuda.synchronize()
    X = scales.cpu().numpy().astype(np.int64) - 127
    deq = MX.mx_dequantize(_codes_to_float(codes), X)
    assert np.isfinite(deq).all()
    assert np.abs(X - X_ref).max() <= 1
    same = (X == X_ref).mean()
    amax = np.abs(ref.reshape(B * N, -1, 32)).max(axis=-1)
    delta = 1e-2 * np.repeat(amax, 32, axis=1)
    # the spacing taken at |v| + delta covers a kernel value one binade up
    bound = _e4m3_half_step(np.abs(ref) + delta, np.repeat(X, 32, axis=1)) * (1 + 2.0 ** -8) + delta
    excess = (np.abs(deq - ref) - bound).max()
    deq_ref = MX.mx_dequantize(P_ref, X_ref)
    half = H * d
    errs = []
    for br in range(2):
        cols = slice(br * half, (br + 1) * half)
        errs.append((rel_err(deq[:, cols], ref[:, cols]), rel_err(deq_ref[:, cols], ref[:, cols])))
    print(f"{case['name']}: exponents equal {same:.4f}, worst excess over the element bound "
          f"{excess:.3e}; rel err (kernel, oracle quantization) softmax {errs[0][0]:.3e}, "
          f"{errs[0][1]:.3e}; linear {errs[1][0]:.3e}, {errs[1][1]:.3e}")
    assert same >= 0.99
    assert excess <= 0.0
    for e_k, e_o in errs:
        assert e_k <= 1.1 * e_o + 2e-3


FP8_SHAPES = [(1, 128, 8), (300, 256, 264), (513, 640, 520), (2048, 6144, 512)]


@pytest.mark.parametrize("M,K,N", FP8_SHAPES, ids=[f"{m}x{k}x{n}" for m, k, n in FP8_SHAPES])
def test_out_proj_mxfp8_product(M, K, N):
    """The FP8 product against the oracle's exact product of the same
    MX-quantized operands (fp32 accumulation and the bf16 output bound the
    difference: 4e-3)."""
    require_gpu()
    _announce(f"out_proj mxfp8 M={M} K={K} N={N}")
    x, w = synth.make_gemm_operands(M, K, N, seed=M + K + N + 1)
    xq, xs = V.mxfp8_quantize(_bf16(x))
    wq, ws = V.mxfp8_quantize(_bf16(w))
    y = V.out_proj_mxfp8(xq, xs, wq, ws)
    torch.cuda.synchronize()
    ref = MX.output_projection_mxfp8(x, w)
    err = rel_err(y.float().cpu().numpy(), ref)
    print(f"out_proj mxfp8 {M}x{K}x{N}: rel err {err:.3e}")
    assert err <= GEMM_TOL


def test_out_proj_mxfp8_768p_sampled_rows():
    require_gpu()
    M, K, N = 60480, 6144, 3072
    _announce(f"out_proj mxfp8 768p M={M} K={K} N={N}")
    x, w = synth.make_gemm_operands(M, K, N, seed=4243)
    xq, xs = V.mxfp8_quantize(_bf16(x))
    wq, ws = V.mxfp8_quantize(_bf16(w))
    y = V.out_proj_mxfp8(xq, xs, wq, ws)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 31, 32, 255, 256, 30000, 30257, M - 193, M - 65, M - 2, M - 1])
    ref = MX.output_projection_mxfp8(x[rows], w)
    got = y[torch.from_numpy(rows).cuda()].float().cpu().numpy()
    err = rel_err(got, ref)
    print(f"out_proj mxfp8 768p sampled rows: rel err {err:.3e}")
    assert err <= GEMM_TOL


@pytest.mark.parametrize("case", PROJ_LAYER_CASES[:2], ids=[c["name"] for c in PROJ_LAYER_CASES[:2]])
def test_layer_with_fp8_projections(case):
    """The layer with FP8 projections against the oracle's FP8 projection of
    its exact gated branches (the softmax kernel quantizes its fp32 branch
    values directly): bound 2e-2, the bf16 layer tolerance."""
    require_gpu()
    case = dict(case)
    dm = case.pop("d_model")
    w = custom(**case)
    _announce(f"layer+proj fp8 {case['name']} d_model={dm}")
    inp = synth.make_inputs(w)
    lay = oracle_layout(w)
    w_o = synth.make_proj_weight(dm, w.heads, w.head_dim, seed=w.seed + 1)
    x2 = O.gated_branches(inp, lay)
    ref = MX.output_projection_mxfp8(x2.reshape(w.batch, w.video_tokens, -1), w_o)
    dev = to_dev(inp, w.dtype)
    L = w.text_tokens
    wq, ws = V.mxfp8_quantize(_bf16(w_o))
    y = V.hybrid_attn_proj_mxfp8(dev["q"], dev["k"], dev["v"], dev["text_k"] if L else None,
                                 dev["text_v"] if L else None, dev["beta"], dev["alpha"],
                                 dev["gate_logits"], wq, ws, frames=w.frames,
                                 tokens_per_frame=w.tokens_per_frame, chunk_frames=w.chunk_frames,
                                 window_chunks=w.window_chunks)
    torch.cuda.synchronize()
    err = rel_err(y.float().cpu().numpy(), ref)
    print(f"{case['name']}: layer + fp8 proj rel err {err:.3e}")
    assert err <= TOL["bf16"]
