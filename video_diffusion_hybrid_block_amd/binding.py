"""ctypes binding of ``libvdn.so`` (the C ABI in ``include/vdn.h``).

Argument marshalling only: shapes are checked against the layout, tensor data
pointers and the current HIP stream are passed to the library, and every step
of the layer runs in the library's gfx950 kernels.  There is no fallback: if
the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "VdnError", "Layout", "lib", "library_path", "version", "validate_layout",
    "num_chunks", "workspace_size", "softmax_workspace_size", "factor_scan_workspace_size",
    "hybrid_attn",
    "softmax_fwd", "softmax_merge_fwd", "softmax_branches_fwd", "softmax_branches_mxfp8",
    "vda_gram", "vda_factor_scan", "vda_branch", "softmax_merge_fwd_vt", "hybrid_attn_noalloc",
    "NOALLOC_SCRATCH_BYTES",
    "merge", "out_proj", "hybrid_attn_proj", "proj_workspace_size", "hybrid_attn_bwd",
    "bwd_workspace_size", "mxfp8_quantize", "out_proj_mxfp8", "hybrid_attn_proj_mxfp8",
    "train_saved_size", "hybrid_attn_fwd_train", "hybrid_attn_bwd_saved",
    "make_layout",
    "EXPORTED_SYMBOLS",
]

VDN_F32, VDN_BF16 = 0, 1
_STATUS = {
    0: "ok", 1: "null argument", 2: "bad shape", 3: "unsupported dtype or head size",
    4: "device pointer not 16-byte aligned", 5: "workspace too small", 6: "HIP launch error",
    7: "layout needs more than the built-in scratch",
}

EXPORTED_SYMBOLS = (
    "vdn_version", "vdn_status_str", "vdn_last_hip_error", "vdn_last_failed_stage",
    "vdn_validate_layout",
    "vdn_num_chunks", "vdn_hybrid_attn_workspace_size", "vdn_hybrid_attn_fwd",
    "vdn_softmax_workspace_size", "vdn_softmax_fwd", "vdn_softmax_merge_fwd", "vdn_vda_gram",
    "vdn_vda_factor_scan_workspace_size",
    "vdn_vda_factor_scan", "vdn_merge", "vdn_softmax_branches_fwd", "vdn_out_proj",
    "vdn_hybrid_attn_proj_workspace_size", "vdn_hybrid_attn_proj_fwd",
    "vdn_hybrid_attn_bwd_workspace_size", "vdn_hybrid_attn_bwd", "vdn_mxfp8_quantize",
    "vdn_out_proj_mxfp8", "vdn_hybrid_attn_proj_mxfp8_workspace_size",
    "vdn_hybrid_attn_proj_mxfp8_fwd", "vdn_softmax_branches_mxfp8_fwd",
    "vdn_hybrid_attn_train_saved_size", "vdn_hybrid_attn_fwd_train", "vdn_hybrid_attn_bwd_saved",
    "vdn_vda_branch", "vdn_hybrid_attn_fwd_noalloc", "vdn_softmax_merge_fwd_vt",
)


class VdnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_STATUS.get(status, status)}")


class Layout(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
        ("head_dim_k", ctypes.c_int32), ("head_dim_v", ctypes.c_int32),
        ("frames", ctypes.c_int32), ("tokens_per_frame", ctypes.c_int32),
        ("chunk_frames", ctypes.c_int32), ("window_chunks", ctypes.c_int32),
        ("anchor_first", ctypes.c_int32), ("anchor_last", ctypes.c_int32),
        ("text_tokens", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float), ("rms_eps", ctypes.c_float),
    ]


def library_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvdn.so")


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with "
                              "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(path)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
        lp = ctypes.POINTER(Layout)
        L.vdn_version.restype = ctypes.c_int
        L.vdn_status_str.restype = ctypes.c_char_p
        L.vdn_status_str.argtypes = [ctypes.c_int]
        L.vdn_last_hip_error.restype = ctypes.c_int
        L.vdn_last_failed_stage.restype = ctypes.c_char_p
        L.vdn_last_failed_stage.argtypes = []
        L.vdn_validate_layout.restype = ctypes.c_int
        L.vdn_validate_layout.argtypes = [lp]
        L.vdn_num_chunks.restype = i32
        L.vdn_num_chunks.argtypes = [lp]
        L.vdn_hybrid_attn_workspace_size.restype = sz
        L.vdn_hybrid_attn_workspace_size.argtypes = [lp]
        L.vdn_vda_factor_scan_workspace_size.restype = sz
        L.vdn_vda_factor_scan_workspace_size.argtypes = [lp]
        L.vdn_hybrid_attn_fwd.restype = ctypes.c_int
        L.vdn_hybrid_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, lp, vp, vp, sz, vp]
        L.vdn_softmax_workspace_size.restype = sz
        L.vdn_softmax_workspace_size.argtypes = [lp]
        L.vdn_softmax_fwd.restype = ctypes.c_int
        L.vdn_softmax_fwd.argtypes = [vp, vp, vp, vp, vp, lp, vp, vp, sz, vp]
        L.vdn_softmax_merge_fwd.restype = ctypes.c_int
        L.vdn_softmax_merge_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, lp, vp, vp, sz, vp]
        L.vdn_vda_gram.restype = ctypes.c_int
        L.vdn_vda_gram.argtypes = [vp, vp, vp, vp, vp, lp, vp, vp, vp]
        L.vdn_vda_factor_scan.restype = ctypes.c_int
        L.vdn_vda_factor_scan.argtypes = [vp, vp, vp, lp, vp, vp, sz, vp]
        L.vdn_merge.restype = ctypes.c_int
        L.vdn_merge.argtypes = [vp, vp, vp, vp, lp, vp, vp]
        L.vdn_softmax_branches_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, lp, vp, vp, sz, vp]
        L.vdn_softmax_branches_fwd.restype = ctypes.c_int
        L.vdn_softmax_branches_mxfp8_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, lp, vp, vp, vp, sz, vp]
        L.vdn_softmax_branches_mxfp8_fwd.restype = ctypes.c_int
        L.vdn_out_proj.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, vp, vp]
        L.vdn_out_proj.restype = ctypes.c_int
        L.vdn_hybrid_attn_proj_workspace_size.argtypes = [lp]
        L.vdn_hybrid_attn_proj_workspace_size.restype = sz
        L.vdn_hybrid_attn_proj_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int32,
                                               lp, vp, vp, sz, vp]
        L.vdn_hybrid_attn_proj_fwd.restype = ctypes.c_int
        L.vdn_hybrid_attn_bwd_workspace_size.argtypes = [lp]
        L.vdn_hybrid_attn_bwd_workspace_size.restype = sz
        L.vdn_hybrid_attn_bwd.argtypes = [vp] * 9 + [lp] + [vp] * 9 + [sz, vp]
        L.vdn_hybrid_attn_bwd.restype = ctypes.c_int
        L.vdn_hybrid_attn_train_saved_size.argtypes = [lp]
        L.vdn_hybrid_attn_train_saved_size.restype = sz
        L.vdn_hybrid_attn_fwd_train.argtypes = [vp] * 8 + [lp, vp, vp, sz, vp]
        L.vdn_hybrid_attn_fwd_train.restype = ctypes.c_int
        L.vdn_hybrid_attn_bwd_saved.argtypes = [vp] * 9 + [lp] + [vp] * 9 + [sz, vp]
        L.vdn_hybrid_attn_bwd_saved.restype = ctypes.c_int
        L.vdn_mxfp8_quantize.argtypes = [vp, ctypes.c_int64, ctypes.c_int32, vp, vp, vp]
        L.vdn_mxfp8_quantize.restype = ctypes.c_int
        L.vdn_out_proj_mxfp8.argtypes = [vp, vp, vp, vp, ctypes.c_int64, ctypes.c_int32,
                                         ctypes.c_int32, vp, vp]
        L.vdn_out_proj_mxfp8.restype = ctypes.c_int
        L.vdn_hybrid_attn_proj_mxfp8_workspace_size.argtypes = [lp]
        L.vdn_hybrid_attn_proj_mxfp8_workspace_size.restype = sz
        L.vdn_hybrid_attn_proj_mxfp8_fwd.argtypes = [vp] * 10 + [ctypes.c_int32, lp, vp, vp, sz, vp]
        L.vdn_hybrid_attn_proj_mxfp8_fwd.restype = ctypes.c_int
        L.vdn_vda_branch.argtypes = [vp] * 6 + [lp, vp, vp, vp, sz, vp]
        L.vdn_softmax_merge_fwd_vt.argtypes = [vp] * 6 + [lp, vp, vp]
        L.vdn_softmax_merge_fwd_vt.restype = ctypes.c_int
        L.vdn_vda_branch.restype = ctypes.c_int
        L.vdn_hybrid_attn_fwd_noalloc.argtypes = [vp] * 8 + [lp, vp, vp]
        L.vdn_hybrid_attn_fwd_noalloc.restype = ctypes.c_int
        _LIB = L
    return _LIB


def version() -> int:
    return lib().vdn_version()


def make_layout(*, batch, heads, head_dim, frames, tokens_per_frame, text_tokens,
                dtype, chunk_frames=5, window_chunks=1, anchor_first=True,
                anchor_last=True, softmax_scale=0.0, rms_eps=0.0) -> Layout:
    if isinstance(dtype, torch.dtype):
        dtype = {torch.bfloat16: VDN_BF16, torch.float32: VDN_F32}.get(dtype, -1)
    elif isinstance(dtype, str):
        dtype = {"bf16": VDN_BF16, "f32": VDN_F32}[dtype]
    return Layout(batch, heads, head_dim, head_dim, frames, tokens_per_frame, chunk_frames,
                  window_chunks, int(bool(anchor_first)), int(bool(anchor_last)), text_tokens,
                  dtype, float(softmax_scale), float(rms_eps))


def _check(status: int, what: str):
    if status != 0:
        if status == 6:
            stage = last_failed_stage()
            if stage:
                what = f"{what} (stage {stage}, hipError {lib().vdn_last_hip_error()})"
        raise VdnError(status, what)


def last_failed_stage():
    """Stage whose launch (or, with VDN_SYNC_DEBUG=1, execution) failed last
    on this thread, or None (``vdn_last_failed_stage``)."""
    s = lib().vdn_last_failed_stage()
    return s.decode() if s else None


def validate_layout(layout: Layout) -> int:
    return lib().vdn_validate_layout(ctypes.byref(layout))


def num_chunks(layout: Layout) -> int:
    return lib().vdn_num_chunks(ctypes.byref(layout))


def workspace_size(layout: Layout) -> int:
    return lib().vdn_hybrid_attn_workspace_size(ctypes.byref(layout))


def softmax_workspace_size(layout: Layout) -> int:
    return lib().vdn_softmax_workspace_size(ctypes.byref(layout))


def factor_scan_workspace_size(layout: Layout) -> int:
    return lib().vdn_vda_factor_scan_workspace_size(ctypes.byref(layout))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _expect(t, shape, dtype, name):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")


def _layout_from(q, text_k, frames, tokens_per_frame, **kw) -> Layout:
    B, N, H, d = q.shape
    if frames * tokens_per_frame != N:
        raise ValueError(f"q has {N} tokens, layout needs frames*tokens_per_frame = "
                         f"{frames * tokens_per_frame}")
    L = 0 if text_k is None else text_k.shape[1]
    return make_layout(batch=B, heads=H, head_dim=d, frames=frames,
                       tokens_per_frame=tokens_per_frame, text_tokens=L, dtype=q.dtype, **kw)


def _workspace(ws, need: int, device, name="workspace"):
    """A caller-provided scratch buffer: a contiguous device uint8 tensor of at
    least `need` bytes (allocated when None)."""
    if ws is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    if ws.dtype != torch.uint8:
        raise ValueError(f"{name}: expected torch.uint8 (view other buffers as bytes)")
    if not ws.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ws.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if ws.numel() < need:
        raise ValueError(f"{name}: {ws.numel()} bytes, {need} needed")
    return ws


def _check_inputs(lay: Layout, q, k, v, text_k, text_v):
    B, H, d = lay.batch, lay.heads, lay.head_dim_k
    N = lay.frames * lay.tokens_per_frame
    dt = q.dtype
    for name, t in (("q", q), ("k", k), ("v", v)):
        _expect(t, (B, N, H, d), dt, name)
    if lay.text_tokens:
        for name, t in (("text_k", text_k), ("text_v", text_v)):
            _expect(t, (B, lay.text_tokens, H, d), dt, name)


def hybrid_attn(q, k, v, text_k, text_v, beta, alpha, gate_logits, *, frames,
                tokens_per_frame, chunk_frames=5, window_chunks=1, anchor_first=True,
                anchor_last=True, softmax_scale=0.0, rms_eps=0.0, out=None,
                workspace=None) -> torch.Tensor:
    """The whole layer (``vdn_hybrid_attn_fwd``).  Tensors are BNHD (see
    ``include/vdn.h``); returns O with the dtype and shape of q."""
    lay = _layout_from(q, text_k, frames, tokens_per_frame, chunk_frames=chunk_frames,
                       window_chunks=window_chunks, anchor_first=anchor_first,
                       anchor_last=anchor_last, softmax_scale=softmax_scale, rms_eps=rms_eps)
    _check(validate_layout(lay), "layout")
    _check_inputs(lay, q, k, v, text_k, text_v)
    B, N, H, _ = q.shape
    L = lay.text_tokens
    _expect(beta, (B, N + L, H), torch.float32, "beta")
    _expect(alpha, (B, frames, H), torch.float32, "alpha")
    _expect(gate_logits, (B, N, H, 2), torch.float32, "gate_logits")
    if out is None:
        out = torch.empty_like(q)
    _expect(out, q.shape, q.dtype, "out")
    need = workspace_size(lay)
    workspace = _workspace(workspace, need, q.device)
    st = lib().vdn_hybrid_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(text_k if L else None), _ptr(text_v if L else None),
        _ptr(beta), _ptr(alpha), _ptr(gate_logits), ctypes.byref(lay), _ptr(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream())
    _check(st, "vdn_hybrid_attn_fwd")
    return out


# VDN_NOALLOC_SCRATCH_BYTES of include/vdn.h
NOALLOC_SCRATCH_BYTES = 64 << 20


def hybrid_attn_noalloc(q, k, v, text_k, text_v, beta, alpha, gate_logits, *, frames,
                        tokens_per_frame, chunk_frames=5, window_chunks=1, anchor_first=True,
                        anchor_last=True, softmax_scale=0.0, rms_eps=0.0,
                        out=None) -> torch.Tensor:
    """The layer without a workspace (``vdn_hybrid_attn_fwd_noalloc``): the
    library's built-in device scratch replaces it, so the call itself
    allocates nothing (``out`` is allocated here when None).  Layouts whose
    workspace exceeds ``NOALLOC_SCRATCH_BYTES`` raise (status 7)."""
    lay = _layout_from(q, text_k, frames, tokens_per_frame, chunk_frames=chunk_frames,
                       window_chunks=window_chunks, anchor_first=anchor_first,
                       anchor_last=anchor_last, softmax_scale=softmax_scale, rms_eps=rms_eps)
    _check(validate_layout(lay), "layout")
    _check_inputs(lay, q, k, v, text_k, text_v)
    B, N, H, _ = q.shape
    L = lay.text_tokens
    _expect(beta, (B, N + L, H), torch.float32, "beta")
    _expect(alpha, (B, frames, H), torch.float32, "alpha")
    _expect(gate_logits, (B, N, H, 2), torch.float32, "gate_logits")
    if out is None:
        out = torch.empty_like(q)
    _expect(out, q.shape, q.dtype, "out")
    st = lib().vdn_hybrid_attn_fwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(text_k if L else None), _ptr(text_v if L else None),
        _ptr(beta), _ptr(alpha), _ptr(gate_logits), ctypes.byref(lay), _ptr(out), _stream())
    _check(st, "vdn_hybrid_attn_fwd_noalloc")
    return out


def softmax_fwd(q, k, v, text_k, text_v, *, frames, tokens_per_frame, chunk_frames=5,
                window_chunks=1, anchor_first=True, anchor_last=True, softmax_scale=0.0,
                out=None, workspace=None) -> torch.Tensor:
    """Softmax branch alone (``vdn_softmax_fwd``)."""
    lay = _layout_from(q, text_k, frames, tokens_per_frame, chunk_frames=chunk_frames,
                       window_chunks=window_chunks, anchor_first=anchor_first,
                       anchor_last=anchor_last, softmax_scale=softmax_scale)
    _check(validate_layout(lay), "layout")
    _check_inputs(lay, q, k, v, text_k, text_v)
    if out is None:
        out = torch.empty_like(q)
    _expect(out, q.shape, q.dtype, "out")
    L = lay.text_tokens
    need = softmax_workspace_size(lay)
    if workspace is not None or need:
        workspace = _workspace(workspace, need, q.device)
    nbytes = 0 if workspace is None else workspace.numel()
    _check(lib().vdn_softmax_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(text_k if L else None),
                                 _ptr(text_v if L else None), ctypes.byref(lay), _ptr(out),
                                 _ptr(workspace), nbytes, _stream()), "vdn_softmax_fwd")
    return out


def softmax_merge_fwd(q, k, v, text_k, text_v, R, gate_logits, *, frames, tokens_per_frame,
                      chunk_frames=5, window_chunks=1, anchor_first=True, anchor_last=True,
                      softmax_scale=0.0, rms_eps=0.0, out=None, workspace=None) -> torch.Tensor:
    """Softmax branch with the merge fused in (``vdn_softmax_merge_fwd``)."""
    lay = _layout_from(q, text_k, frames, tokens_per_frame, chunk_frames=chunk_frames,
                       window_chunks=window_chunks, anchor_first=anchor_first,
                       anchor_last=anchor_last, softmax_scale=softmax_scale, rms_eps=rms_eps)
    _check(validate_layout(lay), "layout")
    _check_inputs(lay, q, k, v, text_k, text_v)
    B, N, H, d = q.shape
    _expect(R, (B, H, num_chunks(lay) + 1, d, d), torch.float32, "R")
    _expect(gate_logits, (B, N, H, 2), torch.float32, "gate_logits")
    if out is None:
        out = torch.empty_like(q)
    _expect(out, q.shape, q.dtype, "out")
    L = lay.text_tokens
    need = softmax_workspace_size(lay)
    if workspace is not None or need:
        workspace = _workspace(workspace, need, q.device)
    nbytes = 0 if workspace is None else workspace.numel()
    _check(lib().vdn_softmax_merge_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(text_k if L else None),
                                       _ptr(text_v if L else None), _ptr(R), _ptr(gate_logits),
                                       ctypes.byref(lay), _ptr(out), _ptr(workspace), nbytes,
                                       _stream()), "vdn_softmax_merge_fwd")
    return out


def softmax_branches_fwd(q, k, v, text_k, text_v, R, gate_logits, *, frames, tokens_per_frame,
                         chunk_frames=5, window_chunks=1, anchor_first=True, anchor_last=True,
                         softmax_scale=0.0, rms_eps=0.0, out=None, workspace=None) -> torch.Tensor:
    """The two gated branches side by side (``vdn_softmax_branches_fwd``):
    returns x2 [B, N, 2, H, d] in q's dtype, softmax branch at index 0."""
    lay = _layout_from(q, text_k, frames, tokens_per_frame, chunk_frames=chunk_frames,
                       window_chunks=window_chunks, anchor_first=anchor_first,
                       anchor_last=anchor_last, softmax_scale=softmax_scale, rms_eps=rms_eps)
    _check(validate_layout(lay), "layout")
    _check_inputs(lay, q, k, v, text_k, text_v)
    B, N, H, d = q.shape
    _expect(R, (B, H, num_chunks(lay) + 1, d, d), torch.float32, "R")
    _expect(gate_logits, (B, N, H, 2), torch.float32, "gate_logits")
    if out is None:
        out = torch.empty((B, N, 2, H, d), dtype=q.dtype, device=q.device)
    _expect(out, (B, N, 2, H, d), q.dtype, "out")
    L = lay.text_tokens
    need = softmax_workspace_size(lay)
    if workspace is not None or need:
        workspace = _workspace(workspace, need, q.device)
    nbytes = 0 if workspace is None else workspace.numel()
    _check(lib().vdn_softmax_branches_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(text_k if L else None),
                                          _ptr(text_v if L else None), _ptr(R),
                                          _ptr(gate_logits), ctypes.byref(lay), _ptr(out),
                                          _ptr(workspace), nbytes, _stream()),
           "vdn_softmax_branches_fwd")
    return out


def softmax_branches_mxfp8(q, k, v, text_k, text_v, R, gate_logits, *, frames, tokens_per_frame,
                           chunk_frames=5, window_chunks=1, anchor_first=True, anchor_last=True,
                           softmax_scale=0.0, rms_eps=0.0, workspace=None):
    """The two gated branches as MXFP8 (``vdn_softmax_branches_mxfp8_fwd``):
    returns (codes uint8 [B*N, 2*H*d], scales uint8 [B*N, 2*H*d/32]); per
    token the softmax branch of every head, then the linear branch."""
    lay = _layout_from(q, text_k, frames, tokens_per_frame, chunk_frames=chunk_frames,
                       window_chunks=window_chunks, anchor_first=anchor_first,
                       anchor_last=anchor_last, softmax_scale=softmax_scale, rms_eps=rms_eps)
    _check(validate_layout(lay), "layout")
    _check_inputs(lay, q, k, v, text_k, text_v)
    B, N, H, d = q.shape
    _expect(R, (B, H, num_chunks(lay) + 1, d, d), torch.float32, "R")
    _expect(gate_logits, (B, N, H, 2), torch.float32, "gate_logits")
    K = 2 * H * d
    codes = torch.empty((B * N, K), dtype=torch.uint8, device=q.device)
    scales = torch.empty((B * N, K // 32), dtype=torch.uint8, device=q.device)
    L = lay.text_tokens
    need = softmax_workspace_size(lay)
    if workspace is not None or need:
        workspace = _workspace(workspace, need, q.device)
    nbytes = 0 if workspace is None else workspace.numel()
    _check(lib().vdn_softmax_branches_mxfp8_fwd(_ptr(q), _ptr(k), _ptr(v),
                                                _ptr(text_k if L else None),
                                                _ptr(text_v if L else None), _ptr(R),
                                                _ptr(gate_logits), ctypes.byref(lay), _ptr(codes),
                                                _ptr(scales), _ptr(workspace), nbytes, _stream()),
           "vdn_softmax_branches_mxfp8_fwd")
    return codes, scales


def out_proj(x, w, out=None) -> torch.Tensor:
    """Output projections as one product (``vdn_out_proj``): x bf16 [..., K],
    w bf16 [N, K]; returns y bf16 [..., N] = x . w^T."""
    if x.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
        raise ValueError("out_proj takes bf16 x and w")
    K = x.shape[-1]
    if w.dim() != 2 or w.shape[1] != K:
        raise ValueError(f"w: expected [N, {K}], got {tuple(w.shape)}")
    N = w.shape[0]
    M = x.numel() // K if K else 0
    _expect(x, x.shape, torch.bfloat16, "x")
    _expect(w, w.shape, torch.bfloat16, "w")
    if out is None:
        out = torch.empty(tuple(x.shape[:-1]) + (N,), dtype=torch.bfloat16, device=x.device)
    _expect(out, tuple(x.shape[:-1]) + (N,), torch.bfloat16, "out")
    _check(lib().vdn_out_proj(_ptr(x), _ptr(w), M, K, N, _ptr(out), _stream()), "vdn_out_proj")
    return out


def proj_workspace_size(layout: Layout) -> int:
    return lib().vdn_hybrid_attn_proj_workspace_size(ctypes.byref(layout))


def hybrid_attn_proj(q, k, v, text_k, text_v, beta, alpha, gate_logits, w_o, *, frames,
                     tokens_per_frame, chunk_frames=5, window_chunks=1, anchor_first=True,
                     anchor_last=True, softmax_scale=0.0, rms_eps=0.0, out=None,
                     workspace=None) -> torch.Tensor:
    """The layer with its separate output projections
    (``vdn_hybrid_attn_proj_fwd``): w_o bf16 [d_model, 2*H*d]; returns y bf16
    [B, N, d_model]."""
    lay = _layout_from(q, text_k, frames, tokens_per_frame, chunk_frames=chunk_frames,
                       window_chunks=window_chunks, anchor_first=anchor_first,
                       anchor_last=anchor_last, softmax_scale=softmax_scale, rms_eps=rms_eps)
    _check(validate_layout(lay), "layout")
    _check_inputs(lay, q, k, v, text_k, text_v)
    B, N, H, d = q.shape
    L = lay.text_tokens
    _expect(beta, (B, N + L, H), torch.float32, "beta")
    _expect(alpha, (B, frames, H), torch.float32, "alpha")
    _expect(gate_logits, (B, N, H, 2), torch.float32, "gate_logits")
    if w_o is None or w_o.dim() != 2 or w_o.shape[1] != 2 * H * d:
        raise ValueError(f"w_o: expected [d_model, {2 * H * d}]")
    _expect(w_o, w_o.shape, q.dtype, "w_o")
    dm = w_o.shape[0]
    if out is None:
        out = torch.empty((B, N, dm), dtype=q.dtype, device=q.device)
    _expect(out, (B, N, dm), q.dtype, "out")
    need = proj_workspace_size(lay)
    workspace = _workspace(workspace, need, q.device)
    st = lib().vdn_hybrid_attn_proj_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(text_k if L else None), _ptr(text_v if L else None),
        _ptr(beta), _ptr(alpha), _ptr(gate_logits), _ptr(w_o), dm, ctypes.byref(lay), _ptr(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream())
    _check(st, "vdn_hybrid_attn_proj_fwd")
    return out


def mxfp8_quantize(x):
    """MXFP8 quantization (``vdn_mxfp8_quantize``) of a bf16 [..., K] tensor:
    returns (codes uint8 [..., K], E8M0 scales uint8 [..., K/32])."""
    if x.dtype != torch.bfloat16:
        raise ValueError("mxfp8_quantize takes bf16")
    K = x.shape[-1]
    _expect(x, x.shape, torch.bfloat16, "x")
    M = x.numel() // K if K else 0
    q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    s = torch.empty(tuple(x.shape[:-1]) + (K // 32,), dtype=torch.uint8, device=x.device)
    _check(lib().vdn_mxfp8_quantize(_ptr(x), M, K, _ptr(q), _ptr(s), _stream()),
           "vdn_mxfp8_quantize")
    return q, s


def out_proj_mxfp8(xq, xs, wq, ws, out=None) -> torch.Tensor:
    """FP8 projection (``vdn_out_proj_mxfp8``) from MXFP8 operands: x codes
    [..., K] + scales [..., K/32], w codes [N, K] + scales [N, K/32]; returns
    bf16 [..., N]."""
    K = xq.shape[-1]
    N = wq.shape[0]
    for name, t in (("xq", xq), ("xs", xs), ("wq", wq), ("ws", ws)):
        _expect(t, t.shape, torch.uint8, name)
    if (tuple(wq.shape) != (N, K) or tuple(ws.shape) != (N, K // 32)
            or tuple(xs.shape) != tuple(xq.shape[:-1]) + (K // 32,)):
        raise ValueError("mxfp8 operand shapes do not match")
    M = xq.numel() // K
    if out is None:
        out = torch.empty(tuple(xq.shape[:-1]) + (N,), dtype=torch.bfloat16, device=xq.device)
    _expect(out, tuple(xq.shape[:-1]) + (N,), torch.bfloat16, "out")
    _check(lib().vdn_out_proj_mxfp8(_ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), M, K, N, _ptr(out),
                                    _stream()), "vdn_out_proj_mxfp8")
    return out


def hybrid_attn_proj_mxfp8(q, k, v, text_k, text_v, beta, alpha, gate_logits, w_q, w_scales, *,
                           frames, tokens_per_frame, chunk_frames=5, window_chunks=1,
                           anchor_first=True, anchor_last=True, softmax_scale=0.0, rms_eps=0.0,
                           out=None, workspace=None) -> torch.Tensor:
    """The layer with FP8 output projections (``vdn_hybrid_attn_proj_mxfp8_fwd``):
    w_q / w_scales from ``mxfp8_quantize(w_o)``; returns y bf16 [B, N, d_model]."""
    lay = _layout_from(q, text_k, frames, tokens_per_frame, chunk_frames=chunk_frames,
                       window_chunks=window_chunks, anchor_first=anchor_first,
                       anchor_last=anchor_last, softmax_scale=softmax_scale, rms_eps=rms_eps)
    _check(validate_layout(lay), "layout")
    _check_inputs(lay, q, k, v, text_k, text_v)
    B, N, H, d = q.shape
    L = lay.text_tokens
    _expect(beta, (B, N + L, H), torch.float32, "beta")
    _expect(alpha, (B, frames, H), torch.float32, "alpha")
    _expect(gate_logits, (B, N, H, 2), torch.float32, "gate_logits")
    K = 2 * H * d
    if w_q.dim() != 2 or w_q.shape[1] != K or w_scales.shape != (w_q.shape[0], K // 32):
        raise ValueError(f"w_q: expected [d_model, {K}] codes and [d_model, {K // 32}] scales")
    _expect(w_q, w_q.shape, torch.uint8, "w_q")
    _expect(w_scales, w_scales.shape, torch.uint8, "w_scales")
    dm = w_q.shape[0]
    if out is None:
        out = torch.empty((B, N, dm), dtype=torch.bfloat16, device=q.device)
    _expect(out, (B, N, dm), torch.bfloat16, "out")
    workspace = _workspace(workspace,
                           lib().vdn_hybrid_attn_proj_mxfp8_workspace_size(ctypes.byref(lay)),
                           q.device)
    st = lib().vdn_hybrid_attn_proj_mxfp8_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(text_k if L else None), _ptr(text_v if L else None),
        _ptr(beta), _ptr(alpha), _ptr(gate_logits), _ptr(w_q), _ptr(w_scales), dm,
        ctypes.byref(lay), _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream())
    _check(st, "vdn_hybrid_attn_proj_mxfp8_fwd")
    return out


def bwd_workspace_size(layout: Layout) -> int:
    return lib().vdn_hybrid_attn_bwd_workspace_size(ctypes.byref(layout))


def hybrid_attn_bwd(q, k, v, text_k, text_v, beta, alpha, gate_logits, dO, *, frames,
                    tokens_per_frame, chunk_frames=5, window_chunks=1, anchor_first=True,
                    anchor_last=True, softmax_scale=0.0, rms_eps=0.0, workspace=None) -> dict:
    """Gradients of the layer (``vdn_hybrid_attn_bwd``) given dO, the
    gradient of the loss with respect to O (dtype and shape of q).  Returns a
    dict of float32 tensors shaped like the inputs: q, k, v, text_k, text_v
    (None without text), beta, alpha, gate_logits."""
    lay = _layout_from(q, text_k, frames, tokens_per_frame, chunk_frames=chunk_frames,
                       window_chunks=window_chunks, anchor_first=anchor_first,
                       anchor_last=anchor_last, softmax_scale=softmax_scale, rms_eps=rms_eps)
    _check(validate_layout(lay), "layout")
    _check_inputs(lay, q, k, v, text_k, text_v)
    B, N, H, d = q.shape
    L = lay.text_tokens
    _expect(beta, (B, N + L, H), torch.float32, "beta")
    _expect(alpha, (B, frames, H), torch.float32, "alpha")
    _expect(gate_logits, (B, N, H, 2), torch.float32, "gate_logits")
    _expect(dO, q.shape, q.dtype, "dO")
    f32 = dict(dtype=torch.float32, device=q.device)
    g = {"q": torch.empty(q.shape, **f32), "k": torch.empty(q.shape, **f32),
         "v": torch.empty(q.shape, **f32),
         "text_k": torch.empty((B, L, H, d), **f32) if L else None,
         "text_v": torch.empty((B, L, H, d), **f32) if L else None,
         "beta": torch.empty((B, N + L, H), **f32), "alpha": torch.empty((B, frames, H), **f32),
         "gate_logits": torch.empty((B, N, H, 2), **f32)}
    need = bwd_workspace_size(lay)
    workspace = _workspace(workspace, need, q.device)
    st = lib().vdn_hybrid_attn_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(text_k if L else None), _ptr(text_v if L else None),
        _ptr(beta), _ptr(alpha), _ptr(gate_logits), _ptr(dO), ctypes.byref(lay), _ptr(g["q"]),
        _ptr(g["k"]), _ptr(g["v"]), _ptr(g["text_k"]), _ptr(g["text_v"]), _ptr(g["beta"]),
        _ptr(g["alpha"]), _ptr(g["gate_logits"]), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream())
    _check(st, "vdn_hybrid_attn_bwd")
    return g


def train_saved_size(layout: Layout) -> int:
    return lib().vdn_hybrid_attn_train_saved_size(ctypes.byref(layout))


def hybrid_attn_fwd_train(q, k, v, text_k, text_v, beta, alpha, gate_logits, *, frames,
                          tokens_per_frame, chunk_frames=5, window_chunks=1, anchor_first=True,
                          anchor_last=True, softmax_scale=0.0, rms_eps=0.0, out=None,
                          saved=None):
    """The layer keeping its residuals (``vdn_hybrid_attn_fwd_train``).
    Returns (O, saved): O as ``hybrid_attn`` returns it and the uint8 buffer
    that ``hybrid_attn_bwd_saved`` consumes."""
    lay = _layout_from(q, text_k, frames, tokens_per_frame, chunk_frames=chunk_frames,
                       window_chunks=window_chunks, anchor_first=anchor_first,
                       anchor_last=anchor_last, softmax_scale=softmax_scale, rms_eps=rms_eps)
    _check(validate_layout(lay), "layout")
    _check_inputs(lay, q, k, v, text_k, text_v)
    B, N, H, _ = q.shape
    L = lay.text_tokens
    _expect(beta, (B, N + L, H), torch.float32, "beta")
    _expect(alpha, (B, frames, H), torch.float32, "alpha")
    _expect(gate_logits, (B, N, H, 2), torch.float32, "gate_logits")
    if out is None:
        out = torch.empty_like(q)
    _expect(out, q.shape, q.dtype, "out")
    saved = _workspace(saved, train_saved_size(lay), q.device, "saved")
    st = lib().vdn_hybrid_attn_fwd_train(
        _ptr(q), _ptr(k), _ptr(v), _ptr(text_k if L else None), _ptr(text_v if L else None),
        _ptr(beta), _ptr(alpha), _ptr(gate_logits), ctypes.byref(lay), _ptr(out), _ptr(saved),
        saved.numel() * saved.element_size(), _stream())
    _check(st, "vdn_hybrid_attn_fwd_train")
    return out, saved


def hybrid_attn_bwd_saved(q, k, v, text_k, text_v, beta, alpha, gate_logits, dO, saved, *,
                          frames, tokens_per_frame, chunk_frames=5, window_chunks=1,
                          anchor_first=True, anchor_last=True, softmax_scale=0.0,
                          rms_eps=0.0) -> dict:
    """Gradients of the layer from the residuals of ``hybrid_attn_fwd_train``
    (``vdn_hybrid_attn_bwd_saved``); same inputs, returns what
    ``hybrid_attn_bwd`` returns.  Consumes ``saved``."""
    lay = _layout_from(q, text_k, frames, tokens_per_frame, chunk_frames=chunk_frames,
                       window_chunks=window_chunks, anchor_first=anchor_first,
                       anchor_last=anchor_last, softmax_scale=softmax_scale, rms_eps=rms_eps)
    _check(validate_layout(lay), "layout")
    _check_inputs(lay, q, k, v, text_k, text_v)
    B, N, H, d = q.shape
    L = lay.text_tokens
    _expect(beta, (B, N + L, H), torch.float32, "beta")
    _expect(alpha, (B, frames, H), torch.float32, "alpha")
    _expect(gate_logits, (B, N, H, 2), torch.float32, "gate_logits")
    _expect(dO, q.shape, q.dtype, "dO")
    f32 = dict(dtype=torch.float32, device=q.device)
    g = {"q": torch.empty(q.shape, **f32), "k": torch.empty(q.shape, **f32),
         "v": torch.empty(q.shape, **f32),
         "text_k": torch.empty((B, L, H, d), **f32) if L else None,
         "text_v": torch.empty((B, L, H, d), **f32) if L else None,
         "beta": torch.empty((B, N + L, H), **f32), "alpha": torch.empty((B, frames, H), **f32),
         "gate_logits": torch.empty((B, N, H, 2), **f32)}
    if saved is None:
        raise ValueError("saved: the buffer hybrid_attn_fwd_train filled is required")
    saved = _workspace(saved, train_saved_size(lay), q.device, "saved")
    st = lib().vdn_hybrid_attn_bwd_saved(
        _ptr(q), _ptr(k), _ptr(v), _ptr(text_k if L else None), _ptr(text_v if L else None),
        _ptr(beta), _ptr(alpha), _ptr(gate_logits), _ptr(dO), ctypes.byref(lay), _ptr(g["q"]),
        _ptr(g["k"]), _ptr(g["v"]), _ptr(g["text_k"]), _ptr(g["text_v"]), _ptr(g["beta"]),
        _ptr(g["alpha"]), _ptr(g["gate_logits"]), _ptr(saved),
        saved.numel() * saved.element_size(), _stream())
    _check(st, "vdn_hybrid_attn_bwd_saved")
    return g


def vda_gram(k, v, text_k, text_v, beta, *, frames, tokens_per_frame, chunk_frames=5,
             window_chunks=1, anchor_first=True, anchor_last=True):
    """Frame statistics (``vdn_vda_gram``): returns (A, B), float32
    [B, H, T+1, d, d] with the text block in slot T."""
    lay = _layout_from(k, text_k, frames, tokens_per_frame, chunk_frames=chunk_frames,
                       window_chunks=window_chunks, anchor_first=anchor_first,
                       anchor_last=anchor_last)
    _check(validate_layout(lay), "layout")
    _check_inputs(lay, k, k, v, text_k, text_v)
    B, N, H, d = k.shape
    L = lay.text_tokens
    _expect(beta, (B, N + L, H), torch.float32, "beta")
    A = torch.empty((B, H, frames + 1, d, d), dtype=torch.float32, device=k.device)
    Bm = torch.empty_like(A)
    _check(lib().vdn_vda_gram(_ptr(k), _ptr(v), _ptr(text_k if L else None),
                              _ptr(text_v if L else None), _ptr(beta), ctypes.byref(lay),
                              _ptr(A), _ptr(Bm), _stream()), "vdn_vda_gram")
    return A, Bm


def vda_factor_scan(A, Bm, alpha, *, dtype, text_tokens, frames, tokens_per_frame,
                    chunk_frames=5, window_chunks=1, anchor_first=True, anchor_last=True):
    """Factor + bidirectional scan (``vdn_vda_factor_scan``).  A is
    overwritten with (I+A)^-1 for the slots the scan uses.  Returns R, float32
    [B, H, nc+1, d, d] (slot nc = text write)."""
    B, H, T1, d, _ = A.shape
    lay = make_layout(batch=B, heads=H, head_dim=d, frames=frames,
                      tokens_per_frame=tokens_per_frame, text_tokens=text_tokens, dtype=dtype,
                      chunk_frames=chunk_frames, window_chunks=window_chunks,
                      anchor_first=anchor_first, anchor_last=anchor_last)
    _check(validate_layout(lay), "layout")
    _expect(A, (B, H, frames + 1, d, d), torch.float32, "A")
    _expect(Bm, (B, H, frames + 1, d, d), torch.float32, "B")
    _expect(alpha, (B, frames, H), torch.float32, "alpha")
    nc = num_chunks(lay)
    R = torch.empty((B, H, nc + 1, d, d), dtype=torch.float32, device=A.device)
    ws = torch.empty(factor_scan_workspace_size(lay), dtype=torch.uint8, device=A.device)
    _check(lib().vdn_vda_factor_scan(_ptr(A), _ptr(Bm), _ptr(alpha), ctypes.byref(lay), _ptr(R),
                                     _ptr(ws), ws.numel(), _stream()), "vdn_vda_factor_scan")
    return R


def vda_branch(k, v, text_k, text_v, beta, alpha, *, frames, tokens_per_frame, chunk_frames=5,
               window_chunks=1, anchor_first=True, anchor_last=True, out=None, vt_out=None,
               want_vt=False, workspace=None):
    """The layer's first stage (``vdn_vda_branch``): returns R, float32
    [B, H, nc+1, d, d] (slot nc = text write), or (R, vt) with ``want_vt`` or
    a ``vt_out`` buffer: vt the V^T copy the layer's softmax reads, bf16
    [B, H, d, T*P + L]."""
    lay = _layout_from(k, text_k, frames, tokens_per_frame, chunk_frames=chunk_frames,
                       window_chunks=window_chunks, anchor_first=anchor_first,
                       anchor_last=anchor_last)
    _check(validate_layout(lay), "layout")
    _check_inputs(lay, k, k, v, text_k, text_v)
    B, N, H, d = k.shape
    L = lay.text_tokens
    _expect(beta, (B, N + L, H), torch.float32, "beta")
    _expect(alpha, (B, frames, H), torch.float32, "alpha")
    nc = num_chunks(lay)
    if out is None:
        out = torch.empty((B, H, nc + 1, d, d), dtype=torch.float32, device=k.device)
    _expect(out, (B, H, nc + 1, d, d), torch.float32, "out")
    if want_vt and vt_out is None:
        vt_out = torch.empty((B, H, d, N + L), dtype=k.dtype, device=k.device)
    if vt_out is not None:
        _expect(vt_out, (B, H, d, N + L), k.dtype, "vt_out")
    workspace = _workspace(workspace, workspace_size(lay), k.device)
    _check(lib().vdn_vda_branch(_ptr(k), _ptr(v), _ptr(text_k if L else None),
                                _ptr(text_v if L else None), _ptr(beta), _ptr(alpha),
                                ctypes.byref(lay), _ptr(out), _ptr(vt_out), _ptr(workspace),
                                workspace.numel(), _stream()), "vdn_vda_branch")
    return (out, vt_out) if vt_out is not None else out


def softmax_merge_fwd_vt(q, k, text_k, vt, R, gate_logits, *, frames, tokens_per_frame,
                         chunk_frames=5, window_chunks=1, anchor_first=True, anchor_last=True,
                         softmax_scale=0.0, rms_eps=0.0, out=None) -> torch.Tensor:
    """The layer's second stage (``vdn_softmax_merge_fwd_vt``): softmax and
    merge from the V^T copy ``vda_branch`` returns."""
    lay = _layout_from(q, text_k, frames, tokens_per_frame, chunk_frames=chunk_frames,
                       window_chunks=window_chunks, anchor_first=anchor_first,
                       anchor_last=anchor_last, softmax_scale=softmax_scale, rms_eps=rms_eps)
    _check(validate_layout(lay), "layout")
    B, N, H, d = q.shape
    L = lay.text_tokens
    _expect(q, (B, N, H, d), q.dtype, "q")
    _expect(k, (B, N, H, d), q.dtype, "k")
    if L:
        _expect(text_k, (B, L, H, d), q.dtype, "text_k")
    _expect(vt, (B, H, d, N + L), q.dtype, "vt")
    _expect(R, (B, H, num_chunks(lay) + 1, d, d), torch.float32, "R")
    _expect(gate_logits, (B, N, H, 2), torch.float32, "gate_logits")
    if out is None:
        out = torch.empty_like(q)
    _expect(out, q.shape, q.dtype, "out")
    _check(lib().vdn_softmax_merge_fwd_vt(_ptr(q), _ptr(k), _ptr(text_k if L else None), _ptr(vt),
                                          _ptr(R), _ptr(gate_logits), ctypes.byref(lay), _ptr(out),
                                          _stream()), "vdn_softmax_merge_fwd_vt")
    return out


def merge(q, o_soft, R, gate_logits, *, frames, tokens_per_frame, chunk_frames=5,
          window_chunks=1, anchor_first=True, anchor_last=True, rms_eps=0.0,
          text_tokens=0, out=None) -> torch.Tensor:
    """Read + RMSNorm + gates + merge (``vdn_merge``); ``out`` may be o_soft."""
    B, N, H, d = q.shape
    lay = make_layout(batch=B, heads=H, head_dim=d, frames=frames,
                      tokens_per_frame=tokens_per_frame, text_tokens=text_tokens, dtype=q.dtype,
                      chunk_frames=chunk_frames, window_chunks=window_chunks,
                      anchor_first=anchor_first, anchor_last=anchor_last, rms_eps=rms_eps)
    _check(validate_layout(lay), "layout")
    _expect(q, (B, frames * tokens_per_frame, H, d), q.dtype, "q")
    _expect(o_soft, q.shape, q.dtype, "o_soft")
    nc = num_chunks(lay)
    _expect(R, (B, H, nc + 1, d, d), torch.float32, "R")
    _expect(gate_logits, (B, N, H, 2), torch.float32, "gate_logits")
    if out is None:
        out = torch.empty_like(q)
    _expect(out, q.shape, q.dtype, "out")
    _check(lib().vdn_merge(_ptr(q), _ptr(o_soft), _ptr(R), _ptr(gate_logits), ctypes.byref(lay),
                           _ptr(out), _stream()), "vdn_merge")
    return out
