"""Host-side checks of the C ABI (CPU only, no kernel launches): exported
symbols, layout validation and error codes, workspace sizing, and the
kernels' frame geometry against the oracle's definitions."""
import ctypes
import itertools
import os
import re
import subprocess

import pytest
import torch

from oracle import vdn_oracle as O
from video_diffusion_hybrid_block_amd import binding as V

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "vdn.h")).read()
    return set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(vdn_\w+)\s*\(", src, flags=re.M))


def test_library_exports_every_declared_symbol():
    lib = V.lib()
    declared = _header_functions()
    assert declared == set(V.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name
    assert V.version() == 100


def _lay(**kw):
    base = dict(batch=1, heads=24, head_dim=128, frames=60, tokens_per_frame=1008,
                text_tokens=512, dtype="bf16")
    base.update(kw)
    return V.make_layout(**base)


def test_validate_layout_error_codes():
    assert V.validate_layout(_lay()) == 0
    assert V.validate_layout(_lay(dtype="f32", head_dim=16)) == 0
    assert V.validate_layout(_lay(frames=0)) == 2
    assert V.validate_layout(_lay(tokens_per_frame=0)) == 2
    assert V.validate_layout(_lay(text_tokens=-1)) == 2
    assert V.validate_layout(_lay(chunk_frames=0)) == 2
    assert V.validate_layout(_lay(window_chunks=-1)) == 2
    assert V.validate_layout(_lay(head_dim=48)) == 3
    assert V.validate_layout(_lay(head_dim=256)) == 3
    bad = _lay()
    bad.dtype = 7
    assert V.validate_layout(bad) == 3
    bad = _lay()
    bad.head_dim_v = 64
    assert V.validate_layout(bad) == 3
    bad = _lay()
    bad.softmax_scale = float("nan")
    assert V.validate_layout(bad) == 2
    assert V.validate_layout(_lay(frames=1 << 20, tokens_per_frame=1 << 12)) == 2
    # token * H * d must stay below 2^31 within one batch element
    assert V.validate_layout(_lay(frames=600, tokens_per_frame=1008)) == 0
    assert V.validate_layout(_lay(frames=700, tokens_per_frame=1008)) == 2
    assert V.lib().vdn_validate_layout(None) == 1


def test_status_strings():
    lib = V.lib()
    for code in range(7):
        assert lib.vdn_status_str(code)
    assert lib.vdn_status_str(99) == b"unknown status"


def test_workspace_size_and_chunks():
    lay = _lay()
    assert V.num_chunks(lay) == 12
    ws = V.workspace_size(lay)
    d2 = 128 * 128 * 4
    assert ws >= 24 * (2 * 61 + 3 * 13) * d2 + 24 * 128 * (60 * 1008 + 512) * 2
    assert V.softmax_workspace_size(lay) == 24 * 128 * (60 * 1008 + 512) * 2
    assert V.softmax_workspace_size(_lay(tokens_per_frame=1001)) == 0   # P not a multiple of 8
    assert V.workspace_size(_lay(frames=120)) > ws
    assert V.workspace_size(_lay(frames=0)) == 0
    assert V.num_chunks(_lay(frames=61)) == 13


@pytest.mark.skipif(torch.cuda.is_available(), reason="argument-error paths are checked without a GPU")
def test_entry_points_reject_bad_arguments_before_launch():
    lib = V.lib()
    lay = _lay(batch=1, heads=1, frames=2, tokens_per_frame=4, text_tokens=0, head_dim=16)
    ok = ctypes.c_void_p(0x10000)         # aligned fake pointers: never dereferenced
    odd = ctypes.c_void_p(0x10004)
    nul = None
    ref = ctypes.byref(lay)
    args = [ok, ok, ok, nul, nul, ok, ok, ok, ref, ok, ok, 1 << 40, nul]
    a = list(args); a[0] = nul
    assert lib.vdn_hybrid_attn_fwd(*a) == 1
    a = list(args); a[9] = odd
    assert lib.vdn_hybrid_attn_fwd(*a) == 4
    a = list(args); a[11] = 16
    assert lib.vdn_hybrid_attn_fwd(*a) == 5
    bad = _lay(head_dim=48)
    a = list(args); a[8] = ctypes.byref(bad)
    assert lib.vdn_hybrid_attn_fwd(*a) == 3
    lay_t = _lay(batch=1, heads=1, frames=2, tokens_per_frame=4, text_tokens=3, head_dim=16)
    a = list(args); a[8] = ctypes.byref(lay_t)
    assert lib.vdn_hybrid_attn_fwd(*a) == 1            # text tensors missing
    assert lib.vdn_softmax_fwd(ok, ok, nul, nul, nul, ref, ok, nul, 0, nul) == 1
    lay_vt = _lay(batch=1, heads=1, frames=2, tokens_per_frame=8, text_tokens=0, head_dim=32)
    assert V.softmax_workspace_size(lay_vt) > 0
    assert lib.vdn_softmax_fwd(ok, ok, ok, nul, nul, ctypes.byref(lay_vt), ok, nul, 0, nul) == 1
    assert lib.vdn_softmax_fwd(ok, ok, ok, nul, nul, ctypes.byref(lay_vt), ok, ok, 16, nul) == 5
    assert lib.vdn_vda_gram(ok, ok, nul, nul, odd, ref, ok, ok, nul) == 4
    assert lib.vdn_vda_factor_scan(ok, ok, ok, ref, ok, ok, 0, nul) == 5
    assert lib.vdn_merge(ok, ok, ok, ok, ref, nul, nul) == 1
    # fused softmax + merge: only the bf16 V^T layouts; then argument checks
    sm = [ok, ok, ok, nul, nul, ok, ok, ctypes.byref(lay_vt), ok, ok, 1 << 40, nul]
    a = list(sm); a[7] = ref                             # f32 d=16: not covered
    assert lib.vdn_softmax_merge_fwd(*a) == 3
    a = list(sm); a[5] = nul
    assert lib.vdn_softmax_merge_fwd(*a) == 1
    a = list(sm); a[6] = odd
    assert lib.vdn_softmax_merge_fwd(*a) == 4
    a = list(sm); a[10] = 16
    assert lib.vdn_softmax_merge_fwd(*a) == 5
    # the layer's VDA branch: same argument checks as the layer
    vb = [ok, ok, nul, nul, ok, ok, ref, ok, nul, ok, 1 << 40, nul]
    a = list(vb); a[7] = nul
    assert lib.vdn_vda_branch(*a) == 1
    a = list(vb); a[5] = odd
    assert lib.vdn_vda_branch(*a) == 4
    a = list(vb); a[10] = 16
    assert lib.vdn_vda_branch(*a) == 5
    a = list(vb); a[6] = ctypes.byref(lay_t)
    assert lib.vdn_vda_branch(*a) == 1                  # text tensors missing
    a = list(vb); a[8] = ok                              # V^T copy: fused layouts only
    assert lib.vdn_vda_branch(*a) == 3
    a = list(vb); a[8] = odd; a[6] = ctypes.byref(lay_vt)
    assert lib.vdn_vda_branch(*a) == 4
    # the second stage from a V^T copy
    sv = [ok, ok, nul, ok, ok, ok, ctypes.byref(lay_vt), ok, nul]
    assert lib.vdn_softmax_merge_fwd_vt(*sv[:6], ref, *sv[7:]) == 3
    a = list(sv); a[3] = nul
    assert lib.vdn_softmax_merge_fwd_vt(*a) == 1
    a = list(sv); a[7] = odd
    assert lib.vdn_softmax_merge_fwd_vt(*a) == 4


def test_backward_and_training_entry_points_reject_bad_arguments_before_launch():
    """vdn_hybrid_attn_bwd, vdn_hybrid_attn_fwd_train and
    vdn_hybrid_attn_bwd_saved return their error codes for one bad argument
    at a time, before any launch (the fake pointers are never used)."""
    lib = V.lib()
    ok = ctypes.c_void_p(0x10000)
    odd = ctypes.c_void_p(0x10004)
    nul = None
    lay = _lay(batch=1, heads=1, frames=2, tokens_per_frame=8, text_tokens=0, head_dim=32)
    ref = ctypes.byref(lay)
    small = ctypes.byref(_lay(batch=1, heads=1, frames=2, tokens_per_frame=8, text_tokens=0,
                              head_dim=16))
    text = ctypes.byref(_lay(batch=1, heads=1, frames=2, tokens_per_frame=8, text_tokens=8,
                             head_dim=32))
    need_bwd = V.bwd_workspace_size(lay)
    need = V.train_saved_size(lay)
    assert need > need_bwd > 0
    assert V.train_saved_size(_lay(frames=0)) == 0
    # forward that keeps its residuals: 8 inputs, layout, o, saved, bytes, stream
    fw = [ok, ok, ok, nul, nul, ok, ok, ok, ref, ok, ok, need, nul]
    for i, val, code in ((9, nul, 1), (10, nul, 1), (0, nul, 1), (9, odd, 4), (10, odd, 4),
                         (11, need - 1, 5), (8, small, 3), (8, text, 1)):
        a = list(fw)
        a[i] = val
        assert lib.vdn_hybrid_attn_fwd_train(*a) == code, (i, code)
    # the two backward calls: 9 inputs, layout, 8 gradients, buffer, bytes, stream
    for fn, size in ((lib.vdn_hybrid_attn_bwd, need_bwd), (lib.vdn_hybrid_attn_bwd_saved, need)):
        bw = [ok, ok, ok, nul, nul, ok, ok, ok, ok, ref,
              ok, ok, ok, nul, nul, ok, ok, ok, ok, size, nul]
        for i, val, code in ((8, nul, 1), (18, nul, 1), (17, nul, 1), (12, odd, 4),
                             (18, odd, 4), (19, size - 1, 5), (9, small, 3), (9, text, 1)):
            a = list(bw)
            a[i] = val
            assert fn(*a) == code, (fn.__name__, i, code)


@pytest.fixture(scope="module")
def geometry_probe(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("geo") / "geometry_probe")
    cmd = ["hipcc", "-O1", "-std=c++17", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "video_diffusion_hybrid_block_amd", "csrc"),
           os.path.join(ROOT, "tests", "geometry_probe.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


def _segments_from_oracle(lay, t):
    """Visible video frames of t as merged token ranges."""
    P = lay.tokens_per_frame
    frames = O.visible_frames(lay, t)
    segs = []
    for f in frames:
        if segs and segs[-1][0] + segs[-1][1] == f * P:
            segs[-1][1] += P
        else:
            segs.append([f * P, P])
    return [tuple(s) for s in segs]


@pytest.mark.parametrize("C,w", [(5, 1), (2, 1), (3, 2), (1, 1), (4, 0), (5, 9)])
def test_kernel_geometry_matches_oracle(geometry_probe, C, w):
    for T, (af, al) in itertools.product(range(1, 31), [(1, 1), (0, 0), (1, 0), (0, 1)]):
        P = 3
        r = subprocess.run([geometry_probe, str(T), str(C), str(w), str(af), str(al), str(P)],
                           capture_output=True, text=True, check=True)
        lines = r.stdout.split("\n")
        lay = O.Layout(batch=1, heads=1, head_dim=16, frames=T, tokens_per_frame=P, text_tokens=0,
                       chunk_frames=C, window_chunks=w, anchor_first=bool(af), anchor_last=bool(al))
        segs = {}
        slots = None
        fold = {}
        for ln in lines:
            f = ln.split()
            if not f:
                continue
            if f[0] == "seg":
                vals = list(map(int, f[2:]))
                segs[int(f[1])] = [tuple(vals[i:i + 2]) for i in range(0, len(vals), 2)]
            elif f[0] == "slots":
                slots = list(map(int, f[1:]))
            elif f[0] in ("fold", "snap"):
                fold.setdefault(f[0], {})[int(f[1])] = list(map(int, f[2:]))
        for t in range(T):
            assert segs[t] == _segments_from_oracle(lay, t), (T, C, w, af, al, t)
        # frames whose statistics the scans need = union of the far sets
        needed = sorted(set().union(*[set(O.far_forward(lay, t)) | set(O.far_backward(lay, t))
                                      for t in range(T)]))
        assert slots == needed + [T], (T, C, w, af, al)
        # backward pass: each chain's fold order, and the state each chunk's
        # snapshot holds = the chunk's far frames, a prefix of that order
        for dr in (0, 1):
            idx = fold["fold"][dr]
            order = sorted((j, f) for f, j in enumerate(idx) if j > 0)
            order = [f for _, f in order]
            assert [j for j, _ in sorted((j, f) for f, j in enumerate(idx) if j > 0)] == \
                list(range(1, len(order) + 1))
            assert order == (sorted(order) if dr == 0 else sorted(order, reverse=True))
            for c in range(lay.num_chunks):
                qf = [t for t in range(c * C, min((c + 1) * C, T)) if t not in O.anchor_frames(lay)]
                if not qf:
                    continue
                far = O.far_forward(lay, qf[0]) if dr == 0 else O.far_backward(lay, qf[0])
                assert order[:fold["snap"][dr][c]] == far, (T, C, w, af, al, dr, c)


def test_projection_entry_points_reject_bad_arguments_before_launch():
    lib = V.lib()
    ok = ctypes.c_void_p(0x10000)         # aligned fake pointers: never dereferenced
    odd = ctypes.c_void_p(0x10004)
    nul = None
    lay_vt = _lay(batch=1, heads=1, frames=2, tokens_per_frame=8, text_tokens=0, head_dim=32)
    lay_16 = _lay(batch=1, heads=1, frames=2, tokens_per_frame=4, text_tokens=0, head_dim=16)
    # gated branches side by side: same coverage and checks as the fused merge
    br = [ok, ok, ok, nul, nul, ok, ok, ctypes.byref(lay_vt), ok, ok, 1 << 40, nul]
    a = list(br); a[7] = ctypes.byref(lay_16)
    assert lib.vdn_softmax_branches_fwd(*a) == 3
    a = list(br); a[8] = nul
    assert lib.vdn_softmax_branches_fwd(*a) == 1
    a = list(br); a[8] = odd
    assert lib.vdn_softmax_branches_fwd(*a) == 4
    a = list(br); a[10] = 16
    assert lib.vdn_softmax_branches_fwd(*a) == 5
    # the product: K a multiple of 64, N a multiple of 8, sizes >= 1
    assert lib.vdn_out_proj(nul, ok, 10, 128, 64, ok, nul) == 1
    assert lib.vdn_out_proj(ok, ok, 0, 128, 64, ok, nul) == 2
    assert lib.vdn_out_proj(ok, ok, 10, 96, 64, ok, nul) == 3
    assert lib.vdn_out_proj(ok, ok, 10, 128, 60, ok, nul) == 3
    assert lib.vdn_out_proj(ok, odd, 10, 128, 64, ok, nul) == 4
    # the layer with projections
    ws = V.proj_workspace_size(lay_vt)
    assert ws > V.workspace_size(lay_vt)
    assert ws - V.workspace_size(lay_vt) >= 2 * 16 * 1 * 32 * 2      # x2: N*2*H*d bf16
    args = [ok, ok, ok, nul, nul, ok, ok, ok, ok, 64, ctypes.byref(lay_vt), ok, ok, 1 << 40, nul]
    a = list(args); a[8] = nul
    assert lib.vdn_hybrid_attn_proj_fwd(*a) == 1
    a = list(args); a[9] = 0
    assert lib.vdn_hybrid_attn_proj_fwd(*a) == 2
    a = list(args); a[9] = 12
    assert lib.vdn_hybrid_attn_proj_fwd(*a) == 3
    a = list(args); a[10] = ctypes.byref(lay_16)
    assert lib.vdn_hybrid_attn_proj_fwd(*a) == 3
    a = list(args); a[11] = odd
    assert lib.vdn_hybrid_attn_proj_fwd(*a) == 4
    a = list(args); a[13] = ws - 256
    assert lib.vdn_hybrid_attn_proj_fwd(*a) == 5


def test_fp8_entry_points_reject_bad_arguments_before_launch():
    lib = V.lib()
    ok = ctypes.c_void_p(0x10000)         # aligned fake pointers: never dereferenced
    odd = ctypes.c_void_p(0x10004)        # 4-byte but not 16-byte aligned
    odd1 = ctypes.c_void_p(0x10001)
    nul = None
    # quantization: K a multiple of 32, M >= 1, x and q 16-byte aligned
    assert lib.vdn_mxfp8_quantize(nul, 4, 64, ok, ok, nul) == 1
    assert lib.vdn_mxfp8_quantize(ok, 0, 64, ok, ok, nul) == 2
    assert lib.vdn_mxfp8_quantize(ok, 4, 48, ok, ok, nul) == 3
    assert lib.vdn_mxfp8_quantize(odd, 4, 64, ok, ok, nul) == 4
    # FP8 product: K a multiple of 128, N of 8; scales 4-byte aligned
    assert lib.vdn_out_proj_mxfp8(ok, nul, ok, ok, 10, 128, 64, ok, nul) == 1
    assert lib.vdn_out_proj_mxfp8(ok, ok, ok, ok, 0, 128, 64, ok, nul) == 2
    assert lib.vdn_out_proj_mxfp8(ok, ok, ok, ok, 10, 96, 64, ok, nul) == 3
    assert lib.vdn_out_proj_mxfp8(ok, ok, ok, ok, 10, 128, 60, ok, nul) == 3
    assert lib.vdn_out_proj_mxfp8(odd, ok, ok, ok, 10, 128, 64, ok, nul) == 4
    assert lib.vdn_out_proj_mxfp8(ok, odd1, ok, ok, 10, 128, 64, ok, nul) == 4
    # branches quantized in the softmax kernel: same coverage as the bf16 branches
    lay_vt = _lay(batch=1, heads=2, frames=2, tokens_per_frame=8, text_tokens=0, head_dim=32)
    lay_16 = _lay(batch=1, heads=1, frames=2, tokens_per_frame=4, text_tokens=0, head_dim=16)
    br = [ok, ok, ok, nul, nul, ok, ok, ctypes.byref(lay_vt), ok, ok, ok, 1 << 40, nul]
    a = list(br); a[7] = ctypes.byref(lay_16)
    assert lib.vdn_softmax_branches_mxfp8_fwd(*a) == 3
    a = list(br); a[9] = nul
    assert lib.vdn_softmax_branches_mxfp8_fwd(*a) == 1
    a = list(br); a[8] = odd
    assert lib.vdn_softmax_branches_mxfp8_fwd(*a) == 4
    a = list(br); a[11] = 16
    assert lib.vdn_softmax_branches_mxfp8_fwd(*a) == 5
    # the layer with FP8 projections: its workspace holds the plan, the codes
    # (N * 2*H*d bytes) and the scales, and no bf16 copy of the branches
    ws = lib.vdn_hybrid_attn_proj_mxfp8_workspace_size(ctypes.byref(lay_vt))
    n_tok, k = 2 * 8, 2 * 2 * 32
    assert ws >= V.workspace_size(lay_vt) + n_tok * k + n_tok * k // 32
    assert ws < V.proj_workspace_size(lay_vt) + n_tok * k + n_tok * k // 32
    args = [ok, ok, ok, nul, nul, ok, ok, ok, ok, ok, 64, ctypes.byref(lay_vt), ok, ok, ws, nul]
    a = list(args); a[8] = nul
    assert lib.vdn_hybrid_attn_proj_mxfp8_fwd(*a) == 1
    a = list(args); a[10] = 0
    assert lib.vdn_hybrid_attn_proj_mxfp8_fwd(*a) == 2
    a = list(args); a[10] = 12
    assert lib.vdn_hybrid_attn_proj_mxfp8_fwd(*a) == 3
    a = list(args); a[11] = ctypes.byref(lay_16)
    assert lib.vdn_hybrid_attn_proj_mxfp8_fwd(*a) == 3
    lay_k64 = _lay(batch=1, heads=1, frames=2, tokens_per_frame=8, text_tokens=0, head_dim=32)
    a = list(args); a[11] = ctypes.byref(lay_k64)          # 2*H*d = 64: not a multiple of 128
    assert lib.vdn_hybrid_attn_proj_mxfp8_fwd(*a) == 3
    a = list(args); a[12] = odd
    assert lib.vdn_hybrid_attn_proj_mxfp8_fwd(*a) == 4
    a = list(args); a[14] = ws - 256
    assert lib.vdn_hybrid_attn_proj_mxfp8_fwd(*a) == 5
