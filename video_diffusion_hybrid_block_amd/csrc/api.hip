// C ABI of the hybrid layer: argument validation, workspace planning and the
// sequence of stage launches.  Everything is enqueued on the caller's stream;
// nothing here allocates device memory or synchronises the host.
#include <dlfcn.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "vdn_internal.h"

using namespace vdn;

namespace {

thread_local int g_last_hip_error = 0;

vdn_status_t hip_status(hipError_t e) {
  if (e == hipSuccess) return VDN_OK;
  g_last_hip_error = (int)e;
  return VDN_ERR_HIP;
}

// Diagnostics, read from the environment on first use; both off by default.
// VDN_SYNC_DEBUG=1: after each stage launch the stream is synchronised and
// checked, so an asynchronous failure is reported by the call (and stage)
// that caused it (skipped on a stream under graph capture).  VDN_ROCTX=1:
// each stage is a roctx range on the calling thread, when the ROCm roctx
// library can be loaded (rocprofv3 --marker-trace records them).
struct Diag {
  bool sync = false;
  int (*push)(const char*) = nullptr;
  int (*pop)() = nullptr;
};

const Diag& diag() {
  static const Diag d = [] {
    Diag r;
    const char* s = getenv("VDN_SYNC_DEBUG");
    r.sync = s && s[0] == '1';
    const char* t = getenv("VDN_ROCTX");
    if (t && t[0] == '1') {
      void* h = dlopen("librocprofiler-sdk-roctx.so.1", RTLD_NOW | RTLD_GLOBAL);
      if (!h) h = dlopen("libroctx64.so.4", RTLD_NOW | RTLD_GLOBAL);
      if (h) {
        r.push = (int (*)(const char*))dlsym(h, "roctxRangePushA");
        r.pop = (int (*)())dlsym(h, "roctxRangePop");
        if (!r.push || !r.pop) r.push = nullptr, r.pop = nullptr;
      }
    }
    return r;
  }();
  return d;
}

thread_local const char* g_failed_stage = nullptr;

// One stage: its launch, bracketed and checked as the diagnostics ask.
template <class F>
hipError_t stage(const char* name, hipStream_t s, F&& launch) {
  const Diag& d = diag();
  if (d.push) d.push(name);
  hipError_t e = launch();
  if (e == hipSuccess && d.sync) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) == hipSuccess && cs == hipStreamCaptureStatusNone) {
      e = hipStreamSynchronize(s);
      if (e == hipSuccess) e = hipGetLastError();
    }
  }
  if (d.pop) d.pop();
  if (e != hipSuccess) g_failed_stage = name;
  return e;
}

#define VDN_STAGE(name, ...) stage(name, stream, [&]() -> hipError_t { return __VA_ARGS__; })

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

vdn_status_t check_layout(const vdn_layout_t* l) {
  if (!l) return VDN_ERR_NULL_ARG;
  if (l->batch < 1 || l->heads < 1 || l->frames < 1 || l->tokens_per_frame < 1 ||
      l->chunk_frames < 1 || l->window_chunks < 0 || l->text_tokens < 0)
    return VDN_ERR_BAD_SHAPE;
  if (l->head_dim_k != l->head_dim_v) return VDN_ERR_UNSUPPORTED;
  const int d = l->head_dim_k;
  if (d != 16 && d != 32 && d != 64 && d != 128) return VDN_ERR_UNSUPPORTED;
  if (l->dtype != VDN_F32 && l->dtype != VDN_BF16) return VDN_ERR_UNSUPPORTED;
  if ((l->anchor_first != 0 && l->anchor_first != 1) || (l->anchor_last != 0 && l->anchor_last != 1))
    return VDN_ERR_BAD_SHAPE;
  if (!(l->softmax_scale >= 0.f) || !isfinite(l->softmax_scale)) return VDN_ERR_BAD_SHAPE;
  if (!(l->rms_eps >= 0.f) || !isfinite(l->rms_eps)) return VDN_ERR_BAD_SHAPE;
  // Index arithmetic inside the kernels uses 32-bit token indices and 32-bit
  // grid sizes; element offsets are 64-bit.
  const long long N = (long long)l->frames * l->tokens_per_frame;
  if (N + l->text_tokens >= (1LL << 31)) return VDN_ERR_BAD_SHAPE;
  // ... and a token's element offset within one batch element, token * H * d,
  // is formed in 32 bits where a key tile's rows are resolved one by one
  if ((N + l->text_tokens) * l->heads * (long long)d >= (1LL << 31)) return VDN_ERR_BAD_SHAPE;
  const long long bh = (long long)l->batch * l->heads;
  if (bh * l->frames * ((l->tokens_per_frame + 63) / 64) >= (1LL << 31)) return VDN_ERR_BAD_SHAPE;
  if (bh * (l->frames + 1) >= (1LL << 31)) return VDN_ERR_BAD_SHAPE;
  return VDN_OK;
}

float eff_scale(const vdn_layout_t& l) {
  return l.softmax_scale > 0.f ? l.softmax_scale : 1.0f / sqrtf((float)l.head_dim_k);
}
float eff_eps(const vdn_layout_t& l) { return l.rms_eps > 0.f ? l.rms_eps : 1e-6f; }

bool text_ok(const vdn_layout_t& l, const void* tk, const void* tv) {
  return l.text_tokens == 0 || (tk != nullptr && tv != nullptr);
}

bool text_aligned(const void* tk, const void* tv) {
  return (!tk || aligned16(tk)) && (!tv || aligned16(tv));
}

// The VDA branch of the layer's forward, up to R (the summed states each
// chunk reads, slot nc the text write) in the plan's buffers.  bf16 layouts
// with d >= 32 take the fused path: statistics and factor in one pass (which
// also writes the softmax's V^T copy when the softmax reads one; *vt_done
// tells), then the scan from the pre-split G planes.  Other layouts take the
// separate gram, factor and scan kernels.
// vt_dst: where the V^T copy goes (the workspace's region for the layer,
// the caller's buffer for vdn_vda_branch, or null: not written).
hipError_t vda_forward(const void* k, const void* v, const void* text_k, const void* text_v,
                       const float* beta, const float* alpha, const vdn_layout_t& l, char* ws,
                       hipStream_t stream, bool* vt_done, float* R_out, void* vt_dst) {
  const Plan p = make_plan(l);
  float* A = (float*)(ws + p.a_off);
  float* B = (float*)(ws + p.b_off);
  float* Sf = (float*)(ws + p.sf_off);
  float* Sb = (float*)(ws + p.sb_off);
  float* R = R_out ? R_out : (float*)(ws + p.r_off);
  *vt_done = false;
  if (l.dtype == VDN_BF16 && l.head_dim_k >= 32) {
    const bool vt = softmax_uses_vt(l) && vt_dst;
    hipError_t e = VDN_STAGE("vda_stats", launch_vda_stats(k, v, text_k, text_v, beta, l, A, B, vt ? vt_dst : nullptr,
                                    stream));
    if (e == hipSuccess) e = VDN_STAGE("scan_split", launch_scan_split(A, B, alpha, l, Sf, Sb, R, stream));
    *vt_done = vt && e == hipSuccess;
    return e;
  }
  hipError_t e = VDN_STAGE("gram", launch_gram(k, v, text_k, text_v, beta, l, false, A, B, stream));
  if (e == hipSuccess) e = VDN_STAGE("factor", launch_factor(A, l, false, stream));
  if (e == hipSuccess) e = VDN_STAGE("scan", launch_scan(A, B, alpha, l, Sf, Sb, R, stream));
  return e;
}

// Host-side checks of the layer's arguments (everything but the workspace).
vdn_status_t check_layer_args(const void* q, const void* k, const void* v, const void* text_k,
                              const void* text_v, const float* beta, const float* alpha,
                              const float* gate_logits, const vdn_layout_t* layout,
                              const void* o) {
  vdn_status_t st = check_layout(layout);
  if (st != VDN_OK) return st;
  if (!q || !k || !v || !beta || !alpha || !gate_logits || !o || !text_ok(*layout, text_k, text_v))
    return VDN_ERR_NULL_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(beta) || !aligned16(alpha) ||
      !aligned16(gate_logits) || !aligned16(o) || !text_aligned(text_k, text_v))
    return VDN_ERR_MISALIGNED;
  return VDN_OK;
}

// The layer on a workspace of at least make_plan(l).total bytes: the VDA
// branch, then the softmax with the merge in its epilogue.
hipError_t layer_forward(const void* q, const void* k, const void* v, const void* text_k,
                         const void* text_v, const float* beta, const float* alpha,
                         const float* gate_logits, const vdn_layout_t& l, void* o, char* ws,
                         hipStream_t stream) {
  const Plan p = make_plan(l);
  float* R = (float*)(ws + p.r_off);
  bool vt_done = false;
  hipError_t e = vda_forward(k, v, text_k, text_v, beta, alpha, l, ws, stream, &vt_done, nullptr,
                             ws + p.vt_off);
  if (e != hipSuccess) return e;
  if (softmax_merge_fusable(l))
    return VDN_STAGE("softmax_merge", launch_softmax_merge(q, k, v, text_k, text_v, R, gate_logits, l, eff_scale(l),
                                eff_eps(l), false, o, ws + p.vt_off, stream, vt_done));
  if (softmax_merge_f32_fusable(l))
    return VDN_STAGE("softmax_merge_f32", launch_softmax_merge_f32(q, k, v, text_k, text_v, R, gate_logits, l,
                                eff_scale(l), eff_eps(l), o, stream));
  e = VDN_STAGE("softmax", launch_softmax(q, k, v, text_k, text_v, l, eff_scale(l), o, ws + p.vt_off, stream));
  if (e == hipSuccess) e = VDN_STAGE("merge", launch_merge(q, o, R, gate_logits, l, eff_eps(l), o, stream));
  return e;
}

}  // namespace

// Workspace of vdn_hybrid_attn_fwd_noalloc.  In host code `scratch` names a
// host-side stand-in, not the device array: the device address comes from
// hipGetSymbolAddress, once per device (each GPU holds its own copy), and
// only that address is handed to kernels.
static __device__ __align__(256) char scratch[VDN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_addr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call there, with that device current).
hipError_t scratch_on_current_device(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = (char*)ptr;
  }
  *out = g_scratch_addr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int vdn_version(void) { return VDN_VERSION; }

const char* vdn_status_str(vdn_status_t s) {
  switch (s) {
    case VDN_OK: return "ok";
    case VDN_ERR_NULL_ARG: return "null argument";
    case VDN_ERR_BAD_SHAPE: return "bad shape";
    case VDN_ERR_UNSUPPORTED: return "unsupported dtype or head size";
    case VDN_ERR_MISALIGNED: return "device pointer not 16-byte aligned";
    case VDN_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case VDN_ERR_HIP: return "HIP launch error";
    case VDN_ERR_SCRATCH_TOO_SMALL: return "layout needs more than the built-in scratch";
  }
  return "unknown status";
}

int vdn_last_hip_error(void) { return g_last_hip_error; }

const char* vdn_last_failed_stage(void) { return g_failed_stage; }

vdn_status_t vdn_validate_layout(const vdn_layout_t* layout) { return check_layout(layout); }

int32_t vdn_num_chunks(const vdn_layout_t* layout) {
  if (check_layout(layout) != VDN_OK) return 0;
  return make_geo(*layout).nc;
}

size_t vdn_hybrid_attn_workspace_size(const vdn_layout_t* layout) {
  if (check_layout(layout) != VDN_OK) return 0;
  return make_plan(*layout).total;
}

size_t vdn_vda_factor_scan_workspace_size(const vdn_layout_t* layout) {
  if (check_layout(layout) != VDN_OK) return 0;
  return scan_ws_bytes(*layout);
}

size_t vdn_softmax_workspace_size(const vdn_layout_t* layout) {
  if (check_layout(layout) != VDN_OK) return 0;
  return softmax_ws_bytes(*layout);
}

vdn_status_t vdn_softmax_fwd(const void* q, const void* k, const void* v, const void* text_k,
                             const void* text_v, const vdn_layout_t* layout, void* o_soft,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  vdn_status_t st = check_layout(layout);
  if (st != VDN_OK) return st;
  if (!q || !k || !v || !o_soft || !text_ok(*layout, text_k, text_v)) return VDN_ERR_NULL_ARG;
  const size_t need = softmax_ws_bytes(*layout);
  if (need > 0 && !workspace) return VDN_ERR_NULL_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o_soft) ||
      !text_aligned(text_k, text_v) || (workspace && !aligned16(workspace)))
    return VDN_ERR_MISALIGNED;
  if (workspace_bytes < need) return VDN_ERR_WORKSPACE_TOO_SMALL;
  return hip_status(VDN_STAGE("softmax", launch_softmax(q, k, v, text_k, text_v, *layout, eff_scale(*layout), o_soft,
                                   workspace, stream)));
}

vdn_status_t vdn_softmax_merge_fwd(const void* q, const void* k, const void* v,
                                   const void* text_k, const void* text_v, const float* R,
                                   const float* gate_logits, const vdn_layout_t* layout, void* o,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  vdn_status_t st = check_layout(layout);
  if (st != VDN_OK) return st;
  if (!softmax_merge_fusable(*layout)) return VDN_ERR_UNSUPPORTED;
  if (!q || !k || !v || !R || !gate_logits || !o || !text_ok(*layout, text_k, text_v))
    return VDN_ERR_NULL_ARG;
  const size_t need = softmax_ws_bytes(*layout);
  if (need > 0 && !workspace) return VDN_ERR_NULL_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(R) || !aligned16(gate_logits) ||
      !aligned16(o) || !text_aligned(text_k, text_v) || (workspace && !aligned16(workspace)))
    return VDN_ERR_MISALIGNED;
  if (workspace_bytes < need) return VDN_ERR_WORKSPACE_TOO_SMALL;
  return hip_status(VDN_STAGE("softmax_merge", launch_softmax_merge(q, k, v, text_k, text_v, R, gate_logits, *layout,
                                         eff_scale(*layout), eff_eps(*layout), false, o, workspace,
                                         stream)));
}

vdn_status_t vdn_softmax_branches_fwd(const void* q, const void* k, const void* v,
                                      const void* text_k, const void* text_v, const float* R,
                                      const float* gate_logits, const vdn_layout_t* layout,
                                      void* x2, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  vdn_status_t st = check_layout(layout);
  if (st != VDN_OK) return st;
  if (!softmax_merge_fusable(*layout)) return VDN_ERR_UNSUPPORTED;
  if (!q || !k || !v || !R || !gate_logits || !x2 || !text_ok(*layout, text_k, text_v))
    return VDN_ERR_NULL_ARG;
  const size_t need = softmax_ws_bytes(*layout);
  if (need > 0 && !workspace) return VDN_ERR_NULL_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(R) || !aligned16(gate_logits) ||
      !aligned16(x2) || !text_aligned(text_k, text_v) || (workspace && !aligned16(workspace)))
    return VDN_ERR_MISALIGNED;
  if (workspace_bytes < need) return VDN_ERR_WORKSPACE_TOO_SMALL;
  return hip_status(VDN_STAGE("softmax_merge", launch_softmax_merge(q, k, v, text_k, text_v, R, gate_logits, *layout,
                                         eff_scale(*layout), eff_eps(*layout), true, x2, workspace,
                                         stream)));
}

vdn_status_t vdn_softmax_branches_mxfp8_fwd(const void* q, const void* k, const void* v,
                                            const void* text_k, const void* text_v,
                                            const float* R, const float* gate_logits,
                                            const vdn_layout_t* layout, void* codes, void* scales,
                                            void* workspace, size_t workspace_bytes,
                                            hipStream_t stream) {
  vdn_status_t st = check_layout(layout);
  if (st != VDN_OK) return st;
  if (!softmax_merge_fusable(*layout)) return VDN_ERR_UNSUPPORTED;
  if (!q || !k || !v || !R || !gate_logits || !codes || !scales ||
      !text_ok(*layout, text_k, text_v))
    return VDN_ERR_NULL_ARG;
  const size_t need = softmax_ws_bytes(*layout);
  if (need > 0 && !workspace) return VDN_ERR_NULL_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(R) || !aligned16(gate_logits) ||
      !aligned16(codes) || !text_aligned(text_k, text_v) || (workspace && !aligned16(workspace)))
    return VDN_ERR_MISALIGNED;
  if (workspace_bytes < need) return VDN_ERR_WORKSPACE_TOO_SMALL;
  return hip_status(VDN_STAGE("softmax_branches_mxfp8", launch_softmax_branches_mxfp8(q, k, v, text_k, text_v, R, gate_logits, *layout,
                                                  eff_scale(*layout), eff_eps(*layout), codes,
                                                  scales, workspace, stream)));
}

vdn_status_t vdn_out_proj(const void* x, const void* w, int64_t M, int32_t K, int32_t N, void* y,
                          hipStream_t stream) {
  if (!x || !w || !y) return VDN_ERR_NULL_ARG;
  if (M < 1 || K < 1 || N < 1) return VDN_ERR_BAD_SHAPE;
  if (!proj_shape_ok(M, K, N)) return VDN_ERR_UNSUPPORTED;
  if ((M + 255) / 256 * ((N + 255) / 256) >= (1LL << 31)) return VDN_ERR_BAD_SHAPE;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return VDN_ERR_MISALIGNED;
  return hip_status(VDN_STAGE("proj", launch_proj(x, w, M, K, N, y, stream)));
}

vdn_status_t vdn_mxfp8_quantize(const void* x, int64_t M, int32_t K, void* q, void* scales,
                                hipStream_t stream) {
  if (!x || !q || !scales) return VDN_ERR_NULL_ARG;
  if (M < 1 || K < 1) return VDN_ERR_BAD_SHAPE;
  if (!mx_quant_shape_ok(M, K)) return VDN_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(q)) return VDN_ERR_MISALIGNED;
  return hip_status(VDN_STAGE("mx_quant", launch_mx_quant(x, M, K, q, scales, stream)));
}

vdn_status_t vdn_out_proj_mxfp8(const void* xq, const void* xs, const void* wq, const void* ws,
                                int64_t M, int32_t K, int32_t N, void* y, hipStream_t stream) {
  if (!xq || !xs || !wq || !ws || !y) return VDN_ERR_NULL_ARG;
  if (M < 1 || K < 1 || N < 1) return VDN_ERR_BAD_SHAPE;
  if (!proj_mxfp8_shape_ok(M, K, N)) return VDN_ERR_UNSUPPORTED;
  if ((M + 255) / 256 * ((N + 255) / 256) >= (1LL << 31)) return VDN_ERR_BAD_SHAPE;
  if (!aligned16(xq) || !aligned16(wq) || !aligned16(y) || ((uintptr_t)xs & 3u) ||
      ((uintptr_t)ws & 3u))
    return VDN_ERR_MISALIGNED;
  return hip_status(VDN_STAGE("proj_mxfp8", launch_proj_mxfp8(xq, xs, wq, ws, M, K, N, y, stream)));
}

vdn_status_t vdn_vda_gram(const void* k, const void* v, const void* text_k, const void* text_v,
                          const float* beta, const vdn_layout_t* layout, float* A_out,
                          float* B_out, hipStream_t stream) {
  vdn_status_t st = check_layout(layout);
  if (st != VDN_OK) return st;
  if (!k || !v || !beta || !A_out || !B_out || !text_ok(*layout, text_k, text_v))
    return VDN_ERR_NULL_ARG;
  if (!aligned16(k) || !aligned16(v) || !aligned16(beta) || !aligned16(A_out) ||
      !aligned16(B_out) || !text_aligned(text_k, text_v))
    return VDN_ERR_MISALIGNED;
  return hip_status(VDN_STAGE("gram", launch_gram(k, v, text_k, text_v, beta, *layout, true, A_out, B_out, stream)));
}

vdn_status_t vdn_vda_factor_scan(float* A_io, const float* B, const float* alpha,
                                 const vdn_layout_t* layout, float* R_out, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  vdn_status_t st = check_layout(layout);
  if (st != VDN_OK) return st;
  if (!A_io || !B || !alpha || !R_out || !workspace) return VDN_ERR_NULL_ARG;
  if (!aligned16(A_io) || !aligned16(B) || !aligned16(alpha) || !aligned16(R_out) ||
      !aligned16(workspace))
    return VDN_ERR_MISALIGNED;
  if (workspace_bytes < scan_ws_bytes(*layout)) return VDN_ERR_WORKSPACE_TOO_SMALL;
  Geo g = make_geo(*layout);
  size_t snaps = align256((size_t)layout->batch * layout->heads * (g.nc + 1) *
                          layout->head_dim_k * layout->head_dim_k * sizeof(float));
  float* Sf = (float*)workspace;
  float* Sb = (float*)((char*)workspace + snaps);
  hipError_t e = VDN_STAGE("factor", launch_factor(A_io, *layout, false, stream));
  if (e != hipSuccess) return hip_status(e);
  return hip_status(VDN_STAGE("scan", launch_scan(A_io, B, alpha, *layout, Sf, Sb, R_out, stream)));
}

vdn_status_t vdn_merge(const void* q, const void* o_soft, const float* R, const float* gate_logits,
                       const vdn_layout_t* layout, void* o, hipStream_t stream) {
  vdn_status_t st = check_layout(layout);
  if (st != VDN_OK) return st;
  if (!q || !o_soft || !R || !gate_logits || !o) return VDN_ERR_NULL_ARG;
  if (!aligned16(q) || !aligned16(o_soft) || !aligned16(R) || !aligned16(gate_logits) ||
      !aligned16(o))
    return VDN_ERR_MISALIGNED;
  return hip_status(VDN_STAGE("merge", launch_merge(q, o_soft, R, gate_logits, *layout, eff_eps(*layout), o, stream)));
}

vdn_status_t vdn_vda_branch(const void* k, const void* v, const void* text_k, const void* text_v,
                            const float* beta, const float* alpha, const vdn_layout_t* layout,
                            float* R_out, void* vt_out, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  vdn_status_t st = check_layout(layout);
  if (st != VDN_OK) return st;
  if (!k || !v || !beta || !alpha || !R_out || !workspace || !text_ok(*layout, text_k, text_v))
    return VDN_ERR_NULL_ARG;
  if (!aligned16(k) || !aligned16(v) || !aligned16(beta) || !aligned16(alpha) ||
      !aligned16(R_out) || !aligned16(workspace) || !text_aligned(text_k, text_v) ||
      (vt_out && !aligned16(vt_out)))
    return VDN_ERR_MISALIGNED;
  if (vt_out && !softmax_merge_fusable(*layout)) return VDN_ERR_UNSUPPORTED;
  const Plan p = make_plan(*layout);
  if (workspace_bytes < p.total) return VDN_ERR_WORKSPACE_TOO_SMALL;
  bool vt_done = false;
  hipError_t e = vda_forward(k, v, text_k, text_v, beta, alpha, *layout, (char*)workspace, stream,
                             &vt_done, R_out, vt_out);
  if (e == hipSuccess && vt_out && !vt_done)   // layouts without the fused statistics pass
    e = VDN_STAGE("transpose", launch_transpose(v, text_v, layout->batch, layout->heads, layout->head_dim_k,
                         layout->frames * layout->tokens_per_frame, layout->text_tokens, vt_out,
                         stream));
  return hip_status(e);
}

vdn_status_t vdn_softmax_merge_fwd_vt(const void* q, const void* k, const void* text_k,
                                      const void* vt, const float* R, const float* gate_logits,
                                      const vdn_layout_t* layout, void* o, hipStream_t stream) {
  vdn_status_t st = check_layout(layout);
  if (st != VDN_OK) return st;
  if (!softmax_merge_fusable(*layout)) return VDN_ERR_UNSUPPORTED;
  if (!q || !k || !vt || !R || !gate_logits || !o || (layout->text_tokens > 0 && !text_k))
    return VDN_ERR_NULL_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(vt) || !aligned16(R) || !aligned16(gate_logits) ||
      !aligned16(o) || (text_k && !aligned16(text_k)))
    return VDN_ERR_MISALIGNED;
  // the kernel reads V only through vt; v / text_v are not needed
  return hip_status(VDN_STAGE("softmax_merge", launch_softmax_merge(q, k, nullptr, text_k, nullptr, R, gate_logits, *layout,
                                         eff_scale(*layout), eff_eps(*layout), false, o,
                                         (void*)vt, stream, true)));
}

vdn_status_t vdn_hybrid_attn_fwd(const void* q, const void* k, const void* v, const void* text_k,
                                 const void* text_v, const float* beta, const float* alpha,
                                 const float* gate_logits, const vdn_layout_t* layout, void* o,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  vdn_status_t st = check_layer_args(q, k, v, text_k, text_v, beta, alpha, gate_logits, layout, o);
  if (st != VDN_OK) return st;
  if (!workspace) return VDN_ERR_NULL_ARG;
  if (!aligned16(workspace)) return VDN_ERR_MISALIGNED;
  if (workspace_bytes < make_plan(*layout).total) return VDN_ERR_WORKSPACE_TOO_SMALL;
  return hip_status(layer_forward(q, k, v, text_k, text_v, beta, alpha, gate_logits, *layout, o,
                                  (char*)workspace, stream));
}

vdn_status_t vdn_hybrid_attn_fwd_noalloc(const void* q, const void* k, const void* v,
                                         const void* text_k, const void* text_v,
                                         const float* beta, const float* alpha,
                                         const float* gate_logits, const vdn_layout_t* layout,
                                         void* o, hipStream_t stream) {
  vdn_status_t st = check_layer_args(q, k, v, text_k, text_v, beta, alpha, gate_logits, layout, o);
  if (st != VDN_OK) return st;
  if (make_plan(*layout).total > (size_t)VDN_NOALLOC_SCRATCH_BYTES) return VDN_ERR_SCRATCH_TOO_SMALL;
  char* ws = nullptr;
  hipError_t e = scratch_on_current_device(&ws);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(layer_forward(q, k, v, text_k, text_v, beta, alpha, gate_logits, *layout, o,
                                  ws, stream));
}

}  // extern "C"

namespace {

// Backward-pass workspace: the forward plan, then the per-step states and
// their gradients, the read-slot gradients, transposed copies and the merge
// backward's outputs.
struct BwdPlan {
  size_t states, dspost, dR, dRp, kt, qt, dost, dos, dlin, nlse, dvec, total;
};

BwdPlan make_bwd_plan(const vdn_layout_t& l) {
  const Plan p = make_plan(l);
  const Geo g = make_geo(l);
  const size_t d = (size_t)l.head_dim_k, bh = (size_t)l.batch * l.heads;
  const size_t N = (size_t)g.T * g.P;
  const size_t mat = d * d * sizeof(float);
  const size_t nl8 = (N + g.L + 7) / 8 * 8, nq8 = (N + 7) / 8 * 8;
  BwdPlan b;
  b.states = p.total;
  b.dspost = align256(b.states + bh * 2 * (g.T + 1) * mat);
  b.dR = align256(b.dspost + bh * 2 * (g.T + 1) * mat);
  b.dRp = align256(b.dR + bh * (g.nc + 1) * mat);
  b.kt = align256(b.dRp + vda_bwd_partial_bytes(l));
  b.qt = align256(b.kt + bh * d * nl8 * 2);
  b.dost = align256(b.qt + bh * d * nq8 * 2);
  b.dos = align256(b.dost + bh * d * nq8 * 2);
  b.dlin = align256(b.dos + (size_t)l.batch * N * l.heads * d * 2);
  b.nlse = align256(b.dlin + (size_t)l.batch * N * l.heads * d * 4);
  b.dvec = align256(b.nlse + bh * N * 4);
  b.total = align256(b.dvec + bh * N * 4);
  return b;
}

// x2 (the gated branches, bf16 [B, T*P, 2, H, d]) follows the layer's plan.
size_t proj_x2_off(const vdn_layout_t& l) { return make_plan(l).total; }
size_t proj_ws_total(const vdn_layout_t& l) {
  return align256(proj_x2_off(l) + (size_t)l.batch * l.frames * l.tokens_per_frame * 2 * l.heads *
                                       l.head_dim_k * 2);
}
bool proj_layer_ok(const vdn_layout_t& l, int32_t d_model) {
  return softmax_merge_fusable(l) &&
         proj_shape_ok((long)l.batch * l.frames * l.tokens_per_frame, 2 * l.heads * l.head_dim_k,
                       d_model);
}

}  // namespace

extern "C" {

}  // extern "C"

namespace {

// The backward after the merge backward (whose dos, dlin, nlse and dvec sit in
// the backward plan's buffers, beside the statistics, factor, read slots and
// per-step states of the forward): transposed copies, the linear branch's
// backward, the statistics backward, then the softmax backward.
hipError_t bwd_tail(const void* q, const void* k, const void* v, const void* text_k,
                    const void* text_v, const float* beta, const float* alpha,
                    const vdn_layout_t& l, float* dq, float* dk, float* dv, float* dtext_k,
                    float* dtext_v, float* dbeta, float* dalpha, char* ws, hipStream_t stream) {
  const Plan p = make_plan(l);
  const BwdPlan bp = make_bwd_plan(l);
  const Geo g = make_geo(l);
  const int N = g.T * g.P;
  float* A = (float*)(ws + p.a_off);
  float* B = (float*)(ws + p.b_off);
  float* R = (float*)(ws + p.r_off);
  float* states = (float*)(ws + bp.states);
  __bf16* dos = (__bf16*)(ws + bp.dos);
  float* dlin = (float*)(ws + bp.dlin);
  float* nlse = (float*)(ws + bp.nlse);
  float* dvec = (float*)(ws + bp.dvec);
  // transposed copies for the softmax backward
  hipError_t e =
      VDN_STAGE("transpose", launch_transpose(k, text_k, l.batch, l.heads, l.head_dim_k, N, g.L, ws + bp.kt, stream));
  if (e == hipSuccess)
    e = VDN_STAGE("transpose", launch_transpose(q, nullptr, l.batch, l.heads, l.head_dim_k, N, 0, ws + bp.qt, stream));
  if (e == hipSuccess)
    e = VDN_STAGE("transpose", launch_transpose(dos, nullptr, l.batch, l.heads, l.head_dim_k, N, 0, ws + bp.dost, stream));
  // linear branch: dq (its part), dA over G, dB over B, dalpha
  if (e == hipSuccess)
    e = VDN_STAGE("vda_bwd", launch_vda_bwd(q, k, v, text_k, text_v, beta, alpha, dlin, R, A, B, states,
                       (float*)(ws + bp.dRp), (float*)(ws + bp.dR), (float*)(ws + bp.dspost), dq,
                       dalpha, l, stream));
  // statistics: dk, dv, dtext_k, dtext_v and dbeta (written)
  if (e == hipSuccess)
    e = VDN_STAGE("gram_bwd", launch_gram_bwd(k, v, text_k, text_v, beta, A, B, dk, dv, dtext_k, dtext_v, dbeta, l,
                        stream));
  // softmax branch: dq, dk, dv, dtext_k, dtext_v (added)
  if (e == hipSuccess)
    e = VDN_STAGE("attn_bwd", launch_attn_bwd(q, k, v, text_k, text_v, dos, nlse, dvec, ws + bp.kt, ws + bp.qt,
                        ws + bp.dost, l, eff_scale(l), dq, dk, dv, dtext_k, dtext_v, stream));
  return e;
}

// Saved residuals of the training pair: the backward plan (whose statistics,
// factor, read slots, per-step states and nlse buffers the training forward
// fills), then O_soft and RMSNorm(R q) (fp32, [B,N,H,d] each) and 1/r
// ([B,H,N] fp32).
struct TrainPlan {
  size_t o_soft, o_lin, rinv, total;
};

TrainPlan make_train_plan(const vdn_layout_t& l) {
  const BwdPlan bp = make_bwd_plan(l);
  const size_t rows = (size_t)l.batch * l.frames * l.tokens_per_frame * l.heads;
  TrainPlan t;
  t.o_soft = bp.total;
  t.o_lin = align256(t.o_soft + rows * l.head_dim_k * 4);
  t.rinv = align256(t.o_lin + rows * l.head_dim_k * 4);
  t.total = align256(t.rinv + rows * 4);
  return t;
}

// Argument checks shared by the two backward entry points.
vdn_status_t check_bwd_args(const void* q, const void* k, const void* v, const void* text_k,
                            const void* text_v, const float* beta, const float* alpha,
                            const float* gate_logits, const void* dO, const vdn_layout_t& l,
                            const float* dq, const float* dk, const float* dv,
                            const float* dtext_k, const float* dtext_v, const float* dbeta,
                            const float* dalpha, const float* dgate_logits, const void* buf) {
  if (!softmax_merge_fusable(l)) return VDN_ERR_UNSUPPORTED;
  const bool txt = l.text_tokens > 0;
  if (!q || !k || !v || !beta || !alpha || !gate_logits || !dO || !dq || !dk || !dv || !dbeta ||
      !dalpha || !dgate_logits || !buf || !text_ok(l, text_k, text_v) ||
      (txt && (!dtext_k || !dtext_v)))
    return VDN_ERR_NULL_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(beta) || !aligned16(alpha) ||
      !aligned16(gate_logits) || !aligned16(dO) || !aligned16(dq) || !aligned16(dk) ||
      !aligned16(dv) || !aligned16(dbeta) || !aligned16(dalpha) || !aligned16(dgate_logits) ||
      !aligned16(buf) || !text_aligned(text_k, text_v) || (dtext_k && !aligned16(dtext_k)) ||
      (dtext_v && !aligned16(dtext_v)))
    return VDN_ERR_MISALIGNED;
  return VDN_OK;
}

}  // namespace

extern "C" {

size_t vdn_hybrid_attn_bwd_workspace_size(const vdn_layout_t* layout) {
  if (check_layout(layout) != VDN_OK) return 0;
  return make_bwd_plan(*layout).total;
}

vdn_status_t vdn_hybrid_attn_bwd(const void* q, const void* k, const void* v, const void* text_k,
                                 const void* text_v, const float* beta, const float* alpha,
                                 const float* gate_logits, const void* dO,
                                 const vdn_layout_t* layout, float* dq, float* dk, float* dv,
                                 float* dtext_k, float* dtext_v, float* dbeta, float* dalpha,
                                 float* dgate_logits, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  vdn_status_t st = check_layout(layout);
  if (st != VDN_OK) return st;
  const vdn_layout_t& l = *layout;
  st = check_bwd_args(q, k, v, text_k, text_v, beta, alpha, gate_logits, dO, l, dq, dk, dv,
                      dtext_k, dtext_v, dbeta, dalpha, dgate_logits, workspace);
  if (st != VDN_OK) return st;
  const BwdPlan bp = make_bwd_plan(l);
  if (workspace_bytes < bp.total) return VDN_ERR_WORKSPACE_TOO_SMALL;
  const Plan p = make_plan(l);
  char* ws = (char*)workspace;
  float* A = (float*)(ws + p.a_off);
  float* B = (float*)(ws + p.b_off);
  float* Sf = (float*)(ws + p.sf_off);
  float* Sb = (float*)(ws + p.sb_off);
  float* R = (float*)(ws + p.r_off);
  float* states = (float*)(ws + bp.states);
  __bf16* dos = (__bf16*)(ws + bp.dos);
  float* dlin = (float*)(ws + bp.dlin);
  float* nlse = (float*)(ws + bp.nlse);
  float* dvec = (float*)(ws + bp.dvec);
  // forward recomputation: statistics, factor, scan (keeping every state)
  hipError_t e = VDN_STAGE("gram", launch_gram(k, v, text_k, text_v, beta, l, false, A, B, stream));
  if (e == hipSuccess) e = VDN_STAGE("factor", launch_factor(A, l, false, stream));
  if (e == hipSuccess) e = VDN_STAGE("scan", launch_scan(A, B, alpha, l, Sf, Sb, R, stream, states));
  // softmax forward with the merge backward in its epilogue
  const EpilogueIO io{(const __bf16*)dO, dgate_logits, dos, dlin, dvec, nlse};
  if (e == hipSuccess)
    e = VDN_STAGE("softmax_merge_bwd", launch_softmax_merge_bwd(q, k, v, text_k, text_v, R, gate_logits, l, eff_scale(l),
                                 eff_eps(l), io, ws + p.vt_off, stream));
  if (e == hipSuccess)
    e = bwd_tail(q, k, v, text_k, text_v, beta, alpha, l, dq, dk, dv, dtext_k, dtext_v, dbeta,
                 dalpha, ws, stream);
  return hip_status(e);
}

size_t vdn_hybrid_attn_train_saved_size(const vdn_layout_t* layout) {
  if (check_layout(layout) != VDN_OK) return 0;
  return make_train_plan(*layout).total;
}

vdn_status_t vdn_hybrid_attn_fwd_train(const void* q, const void* k, const void* v,
                                       const void* text_k, const void* text_v, const float* beta,
                                       const float* alpha, const float* gate_logits,
                                       const vdn_layout_t* layout, void* o, void* saved,
                                       size_t saved_bytes, hipStream_t stream) {
  vdn_status_t st = check_layout(layout);
  if (st != VDN_OK) return st;
  const vdn_layout_t& l = *layout;
  if (!softmax_merge_fusable(l)) return VDN_ERR_UNSUPPORTED;
  if (!q || !k || !v || !beta || !alpha || !gate_logits || !o || !saved ||
      !text_ok(l, text_k, text_v))
    return VDN_ERR_NULL_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(beta) || !aligned16(alpha) ||
      !aligned16(gate_logits) || !aligned16(o) || !aligned16(saved) ||
      !text_aligned(text_k, text_v))
    return VDN_ERR_MISALIGNED;
  const TrainPlan tp = make_train_plan(l);
  if (saved_bytes < tp.total) return VDN_ERR_WORKSPACE_TOO_SMALL;
  const Plan p = make_plan(l);
  const BwdPlan bp = make_bwd_plan(l);
  char* ws = (char*)saved;
  float* A = (float*)(ws + p.a_off);
  float* B = (float*)(ws + p.b_off);
  float* R = (float*)(ws + p.r_off);
  hipError_t e = VDN_STAGE("gram", launch_gram(k, v, text_k, text_v, beta, l, false, A, B, stream));
  if (e == hipSuccess) e = VDN_STAGE("factor", launch_factor(A, l, false, stream));
  if (e == hipSuccess)
    e = VDN_STAGE("scan", launch_scan(A, B, alpha, l, (float*)(ws + p.sf_off), (float*)(ws + p.sb_off), R, stream,
                    (float*)(ws + bp.states)));
  EpilogueIO io{};
  io.nlse = (float*)(ws + bp.nlse);
  io.o_soft = (float*)(ws + tp.o_soft);
  io.o_lin = (float*)(ws + tp.o_lin);
  io.rinv = (float*)(ws + tp.rinv);
  if (e == hipSuccess)
    e = VDN_STAGE("softmax_merge_train", launch_softmax_merge_train(q, k, v, text_k, text_v, R, gate_logits, l, eff_scale(l),
                                   eff_eps(l), o, io, ws + p.vt_off, stream));
  return hip_status(e);
}

vdn_status_t vdn_hybrid_attn_bwd_saved(const void* q, const void* k, const void* v,
                                       const void* text_k, const void* text_v, const float* beta,
                                       const float* alpha, const float* gate_logits,
                                       const void* dO, const vdn_layout_t* layout, float* dq,
                                       float* dk, float* dv, float* dtext_k, float* dtext_v,
                                       float* dbeta, float* dalpha, float* dgate_logits,
                                       void* saved, size_t saved_bytes, hipStream_t stream) {
  vdn_status_t st = check_layout(layout);
  if (st != VDN_OK) return st;
  const vdn_layout_t& l = *layout;
  st = check_bwd_args(q, k, v, text_k, text_v, beta, alpha, gate_logits, dO, l, dq, dk, dv,
                      dtext_k, dtext_v, dbeta, dalpha, dgate_logits, saved);
  if (st != VDN_OK) return st;
  const TrainPlan tp = make_train_plan(l);
  if (saved_bytes < tp.total) return VDN_ERR_WORKSPACE_TOO_SMALL;
  const BwdPlan bp = make_bwd_plan(l);
  char* ws = (char*)saved;
  hipError_t e = VDN_STAGE("merge_bwd_saved", launch_merge_bwd_saved(
      dO, gate_logits, (const float*)(ws + tp.o_soft), (const float*)(ws + tp.o_lin),
      (const float*)(ws + tp.rinv), l, dgate_logits, ws + bp.dos, (float*)(ws + bp.dlin),
      (float*)(ws + bp.dvec), stream));
  if (e == hipSuccess)
    e = bwd_tail(q, k, v, text_k, text_v, beta, alpha, l, dq, dk, dv, dtext_k, dtext_v, dbeta,
                 dalpha, ws, stream);
  return hip_status(e);
}

// Workspace of the layer with FP8 projections: the layer's plan (VDA
// buffers, V^T copy), then the MXFP8 codes [M][K] and scales [M][K/32] of the
// two gated branches.
static size_t fp8_codes_off(const vdn_layout_t& l) { return align256(make_plan(l).total); }
static size_t fp8_scales_off(const vdn_layout_t& l) {
  const size_t M = (size_t)l.batch * l.frames * l.tokens_per_frame;
  return align256(fp8_codes_off(l) + M * 2 * l.heads * l.head_dim_k);
}

size_t vdn_hybrid_attn_proj_mxfp8_workspace_size(const vdn_layout_t* layout) {
  if (check_layout(layout) != VDN_OK) return 0;
  const vdn_layout_t& l = *layout;
  const size_t M = (size_t)l.batch * l.frames * l.tokens_per_frame;
  const size_t K = 2 * (size_t)l.heads * l.head_dim_k;
  return align256(fp8_scales_off(l) + M * (K / 32));
}

vdn_status_t vdn_hybrid_attn_proj_mxfp8_fwd(const void* q, const void* k, const void* v,
                                            const void* text_k, const void* text_v,
                                            const float* beta, const float* alpha,
                                            const float* gate_logits, const void* w_q,
                                            const void* w_scales, int32_t d_model,
                                            const vdn_layout_t* layout, void* y, void* workspace,
                                            size_t workspace_bytes, hipStream_t stream) {
  vdn_status_t st = check_layout(layout);
  if (st != VDN_OK) return st;
  if (d_model < 1) return VDN_ERR_BAD_SHAPE;
  const vdn_layout_t& l = *layout;
  const long M = (long)l.batch * l.frames * l.tokens_per_frame;
  const int K = 2 * l.heads * l.head_dim_k;
  if (!softmax_merge_fusable(l) || !proj_mxfp8_shape_ok(M, K, d_model)) return VDN_ERR_UNSUPPORTED;
  if ((M + 255) / 256 * ((d_model + 255) / 256) >= (1LL << 31)) return VDN_ERR_BAD_SHAPE;
  if (!q || !k || !v || !beta || !alpha || !gate_logits || !w_q || !w_scales || !y ||
      !workspace || !text_ok(l, text_k, text_v))
    return VDN_ERR_NULL_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(beta) || !aligned16(alpha) ||
      !aligned16(gate_logits) || !aligned16(w_q) || ((uintptr_t)w_scales & 3u) || !aligned16(y) ||
      !aligned16(workspace) || !text_aligned(text_k, text_v))
    return VDN_ERR_MISALIGNED;
  if (workspace_bytes < vdn_hybrid_attn_proj_mxfp8_workspace_size(layout))
    return VDN_ERR_WORKSPACE_TOO_SMALL;
  const Plan p = make_plan(l);
  char* ws = (char*)workspace;
  float* R = (float*)(ws + p.r_off);
  char* xq = ws + fp8_codes_off(l);
  char* xs = ws + fp8_scales_off(l);
  bool vt_done = false;
  hipError_t e = vda_forward(k, v, text_k, text_v, beta, alpha, l, ws, stream, &vt_done, nullptr,
                             ws + p.vt_off);
  if (e == hipSuccess)
    e = VDN_STAGE("softmax_branches_mxfp8", launch_softmax_branches_mxfp8(q, k, v, text_k, text_v, R, gate_logits, l, eff_scale(l),
                                      eff_eps(l), xq, xs, ws + p.vt_off, stream, vt_done));
  if (e == hipSuccess) e = VDN_STAGE("proj_mxfp8", launch_proj_mxfp8(xq, xs, w_q, w_scales, M, K, d_model, y, stream));
  return hip_status(e);
}

size_t vdn_hybrid_attn_proj_workspace_size(const vdn_layout_t* layout) {
  if (check_layout(layout) != VDN_OK) return 0;
  return proj_ws_total(*layout);
}

vdn_status_t vdn_hybrid_attn_proj_fwd(const void* q, const void* k, const void* v,
                                      const void* text_k, const void* text_v, const float* beta,
                                      const float* alpha, const float* gate_logits,
                                      const void* w_o, int32_t d_model,
                                      const vdn_layout_t* layout, void* y, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  vdn_status_t st = check_layout(layout);
  if (st != VDN_OK) return st;
  if (d_model < 1) return VDN_ERR_BAD_SHAPE;
  const vdn_layout_t& l = *layout;
  if (!proj_layer_ok(l, d_model)) return VDN_ERR_UNSUPPORTED;
  const long M = (long)l.batch * l.frames * l.tokens_per_frame;
  if ((M + 255) / 256 * ((d_model + 255) / 256) >= (1LL << 31)) return VDN_ERR_BAD_SHAPE;
  if (!q || !k || !v || !beta || !alpha || !gate_logits || !w_o || !y || !workspace ||
      !text_ok(l, text_k, text_v))
    return VDN_ERR_NULL_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(beta) || !aligned16(alpha) ||
      !aligned16(gate_logits) || !aligned16(w_o) || !aligned16(y) || !aligned16(workspace) ||
      !text_aligned(text_k, text_v))
    return VDN_ERR_MISALIGNED;
  if (workspace_bytes < proj_ws_total(l)) return VDN_ERR_WORKSPACE_TOO_SMALL;
  const Plan p = make_plan(l);
  char* ws = (char*)workspace;
  float* R = (float*)(ws + p.r_off);
  void* x2 = ws + proj_x2_off(l);
  bool vt_done = false;
  hipError_t e = vda_forward(k, v, text_k, text_v, beta, alpha, l, ws, stream, &vt_done, nullptr,
                             ws + p.vt_off);
  if (e == hipSuccess)
    e = VDN_STAGE("softmax_merge", launch_softmax_merge(q, k, v, text_k, text_v, R, gate_logits, l, eff_scale(l), eff_eps(l),
                             true, x2, ws + p.vt_off, stream, vt_done));
  if (e == hipSuccess) e = VDN_STAGE("proj", launch_proj(x2, w_o, M, 2 * l.heads * l.head_dim_k, d_model, y, stream));
  return hip_status(e);
}

}  // extern "C"
