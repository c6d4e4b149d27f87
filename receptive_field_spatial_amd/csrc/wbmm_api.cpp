// C ABI of libwbmm: argument validation (host only, before anything is enqueued), the thread-local
// error message, and dispatch to the kernel launchers.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/wbmm.h"
#include "wbmm_launch.hpp"

#define WBMM_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_err;
thread_local hipEvent_t g_ev_before = nullptr, g_ev_after = nullptr;

wbmm_status fail(wbmm_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

wbmm_status ok() {
  g_err.clear();
  return WBMM_OK;
}

wbmm_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(WBMM_E_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

constexpr int kMaxW = 32;
constexpr long long kMaxDim = 1 << 20;
constexpr long long kMaxElems = 1ll << 38;

bool valid_dtype(int dt) { return dt == WBMM_F32 || dt == WBMM_BF16; }
bool valid_layout(int l) { return l == WBMM_NCHW || l == WBMM_NHWC; }
size_t dtype_size(int dt) { return dt == WBMM_BF16 ? 2 : 4; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Byte ranges [p, p + n) and [q, q + m) intersect.
bool overlaps(const void* p, size_t n, const void* q, size_t m) {
  if (!p || !q || n == 0 || m == 0) return false;
  const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
  return a < b + m && b < a + n;
}

wbmm_status check_map(int B, int C, int H, int W, int w, int layout) {
  if (w < 1 || w > kMaxW) return fail(WBMM_E_INVALID, "window size w=%d outside [1, %d]", w, kMaxW);
  if (B < 1 || C < 1 || H < 1 || W < 1)
    return fail(WBMM_E_INVALID, "sizes must be >= 1 (B=%d C=%d H=%d W=%d)", B, C, H, W);
  if (C > 65535) return fail(WBMM_E_UNSUPPORTED, "C=%d exceeds 65535", C);
  if (B > kMaxDim || H > kMaxDim || W > kMaxDim)
    return fail(WBMM_E_UNSUPPORTED, "a dimension exceeds 2^20");
  const long long Hp = (H + w - 1) / w * (long long)w, Wp = (W + w - 1) / w * (long long)w;
  if ((long long)B * C * Hp * Wp > kMaxElems) return fail(WBMM_E_UNSUPPORTED, "map too large");
  if ((long long)B * (Hp / w) * (Wp / w) >= (1ll << 31))
    return fail(WBMM_E_UNSUPPORTED, "too many windows per channel");
  if (!valid_layout(layout)) return fail(WBMM_E_INVALID, "unknown layout %d", layout);
  return WBMM_OK;
}

}  // namespace

namespace wbmm {
void take_main_events(hipEvent_t* before, hipEvent_t* after) {
  *before = g_ev_before;
  *after = g_ev_after;
  g_ev_before = g_ev_after = nullptr;  // one call only
}
}  // namespace wbmm

WBMM_API int wbmm_abi_version(void) { return WBMM_ABI_VERSION; }

WBMM_API wbmm_status wbmm_set_launch_events(void* before, void* after) {
  if ((before == nullptr) != (after == nullptr))
    return fail(WBMM_E_INVALID, "give both events or neither");
  g_ev_before = (hipEvent_t)before;
  g_ev_after = (hipEvent_t)after;
  return ok();
}

WBMM_API const char* wbmm_last_error(void) { return g_err.c_str(); }

WBMM_API wbmm_status wbmm_build_index(int w, int32_t* idx, void* stream) {
  if (w < 1 || w > kMaxW) return fail(WBMM_E_INVALID, "window size w=%d outside [1, %d]", w, kMaxW);
  if (!idx) return fail(WBMM_E_INVALID, "idx is NULL");
  if (!aligned(idx, 4)) return fail(WBMM_E_UNSUPPORTED, "idx not 4-byte aligned");
  return hip_status(wbmm::launch_build_index(w, idx, (hipStream_t)stream), "wbmm_build_index");
}

WBMM_API wbmm_status wbmm_build_matrix(const void* T, int C, int w, int dtype, void* M,
                                       void* stream) {
  if (w < 1 || w > kMaxW) return fail(WBMM_E_INVALID, "window size w=%d outside [1, %d]", w, kMaxW);
  if (C < 1) return fail(WBMM_E_INVALID, "C=%d must be >= 1", C);
  if (!valid_dtype(dtype)) return fail(WBMM_E_INVALID, "unknown dtype %d", dtype);
  if (!T || !M) return fail(WBMM_E_INVALID, "T and M must be non-NULL");
  const size_t es = dtype_size(dtype);
  if (!aligned(T, es) || !aligned(M, es)) return fail(WBMM_E_UNSUPPORTED, "misaligned pointer");
  const size_t L = (size_t)(2 * w - 1) * (2 * w - 1), d = (size_t)w * w;
  if (overlaps(T, (size_t)C * L * es, M, (size_t)C * d * d * es))
    return fail(WBMM_E_INVALID, "M overlaps T");
  return hip_status(wbmm::launch_build_matrix(T, C, w, dtype == WBMM_BF16, M, (hipStream_t)stream),
                    "wbmm_build_matrix");
}

WBMM_API wbmm_status wbmm_fold_hier(const void* M_in, const void* T_sub, int C, int w, int s,
                                    int dtype, void* M_out, void* stream) {
  if (w < 1 || w > kMaxW) return fail(WBMM_E_INVALID, "window size w=%d outside [1, %d]", w, kMaxW);
  if (C < 1) return fail(WBMM_E_INVALID, "C=%d must be >= 1", C);
  if (s < 1 || s >= w || w % s != 0)
    return fail(WBMM_E_INVALID, "sub-window s=%d must divide w=%d with 1 <= s < w", s, w);
  if (!valid_dtype(dtype)) return fail(WBMM_E_INVALID, "unknown dtype %d", dtype);
  if (!M_in || !T_sub || !M_out) return fail(WBMM_E_INVALID, "NULL pointer");
  const size_t es = dtype_size(dtype);
  if (!aligned(M_in, es) || !aligned(T_sub, es) || !aligned(M_out, es))
    return fail(WBMM_E_UNSUPPORTED, "misaligned pointer");
  const size_t mbytes = (size_t)C * w * w * w * w * es;
  if (M_in != M_out && overlaps(M_in, mbytes, M_out, mbytes))
    return fail(WBMM_E_INVALID, "M_out partially overlaps M_in");
  const size_t tbytes = (size_t)C * (2 * s - 1) * (2 * s - 1) * es;
  if (overlaps(T_sub, tbytes, M_out, mbytes)) return fail(WBMM_E_INVALID, "M_out overlaps T_sub");
  return hip_status(
      wbmm::launch_fold(M_in, T_sub, C, w, s, dtype == WBMM_BF16, M_out, (hipStream_t)stream),
      "wbmm_fold_hier");
}

namespace {

wbmm_status check_forward(const wbmm::FwdRequest& r, int in_dtype, int out_dtype) {
  wbmm_status st = check_map(r.B, r.C, r.H, r.W, r.w, r.layout);
  if (st != WBMM_OK) return st;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return fail(WBMM_E_INVALID, "unknown dtype (in %d, out %d)", in_dtype, out_dtype);
  if (!r.x || !r.y) return fail(WBMM_E_INVALID, "x and y must be non-NULL");
  if ((r.T == nullptr) == (r.M == nullptr))
    return fail(WBMM_E_INVALID, "exactly one of T (table) and M (cached matrix) must be given");
  const size_t ies = dtype_size(in_dtype), oes = dtype_size(out_dtype);
  if (!aligned(r.x, ies) || (r.T && !aligned(r.T, ies)) || (r.M && !aligned(r.M, ies)) ||
      !aligned(r.y, oes) || (r.zsave && !aligned(r.zsave, oes)) || (r.mixw && !aligned(r.mixw, 4)))
    return fail(WBMM_E_UNSUPPORTED, "pointer not aligned to its element size");
  const size_t elems = (size_t)r.B * r.C * r.H * r.W;
  const size_t d = (size_t)r.w * r.w, L = (size_t)(2 * r.w - 1) * (2 * r.w - 1);
  const size_t ybytes = elems * oes;
  if (overlaps(r.y, ybytes, r.x, elems * ies)) return fail(WBMM_E_INVALID, "y overlaps x");
  if (overlaps(r.y, ybytes, r.T, (size_t)r.C * L * ies)) return fail(WBMM_E_INVALID, "y overlaps T");
  if (overlaps(r.y, ybytes, r.M, (size_t)r.C * d * d * ies))
    return fail(WBMM_E_INVALID, "y overlaps M");
  if (overlaps(r.y, ybytes, r.mixw, (size_t)r.C * 9 * 4))
    return fail(WBMM_E_INVALID, "y overlaps mix_w");
  if (overlaps(r.y, ybytes, r.zsave, ybytes)) return fail(WBMM_E_INVALID, "y overlaps z_save");
  if (r.zsave && overlaps(r.zsave, ybytes, r.x, elems * ies))
    return fail(WBMM_E_INVALID, "z_save overlaps x");
  if (!wbmm::forward_plan_ok(r))
    return fail(WBMM_E_UNSUPPORTED, "no launch shape fits this problem (w=%d)", r.w);
  return WBMM_OK;
}

wbmm::FwdRequest make_fwd(int B, int C, int H, int W, int w, int layout, int in_dtype,
                          int out_dtype, const void* x, const void* T, const void* M,
                          const float* mix_w, void* z_save, void* y, void* ws, size_t ws_bytes) {
  wbmm::FwdRequest r{};
  r.B = B; r.C = C; r.H = H; r.W = W; r.w = w; r.layout = layout;
  r.in_bf16 = in_dtype == WBMM_BF16;
  r.out_bf16 = out_dtype == WBMM_BF16;
  r.x = x; r.T = T; r.M = M; r.mixw = mix_w; r.zsave = z_save; r.y = y;
  r.ws = ws; r.ws_bytes = ws_bytes;
  return r;
}

}  // namespace

namespace {

bool offsets_ok(int w, int oy, int ox) { return oy >= 0 && ox >= 0 && oy < w && ox < w; }

size_t forward_ws_bytes(int B, int C, int H, int W, int w, int oy, int ox, int layout, int has_mix,
                        int has_z_save) {
  if (check_map(B, C, H + oy, W + ox, w, layout) != WBMM_OK || !offsets_ok(w, oy, ox)) return 0;
  static const float dummy = 0.f;
  wbmm::FwdRequest r = make_fwd(B, C, H, W, w, layout, WBMM_F32, WBMM_F32, &dummy, &dummy, nullptr,
                                has_mix ? &dummy : nullptr, has_z_save ? (void*)&dummy : nullptr,
                                (void*)&dummy, nullptr, 0);
  r.oy = oy;
  r.ox = ox;
  if (!wbmm::forward_plan_ok(r)) return 0;
  // the dtypes and the operand kind are not arguments: the largest need over fp32 / bf16 inputs
  // and outputs, with a table or a cached matrix
  size_t need = 0;
  for (int cached = 0; cached < 2; ++cached)
    for (int ib = 0; ib < 2; ++ib)
      for (int ob = 0; ob < 2; ++ob) {
        r.T = cached ? nullptr : (const void*)&dummy;
        r.M = cached ? (const void*)&dummy : nullptr;
        r.in_bf16 = ib;
        r.out_bf16 = ob;
        if (cached && !wbmm::forward_plan_ok(r)) continue;
        const size_t n = wbmm::forward_workspace(r);
        if (n > need) need = n;
      }
  return need;
}

wbmm_status forward_call(int B, int C, int H, int W, int w, int oy, int ox, int layout,
                         int in_dtype, int out_dtype, const void* x, const void* T, const void* M,
                         const float* mix_w, void* z_save, void* y, void* workspace,
                         size_t workspace_bytes, void* stream, const char* name) {
  if (!offsets_ok(w, oy, ox))
    return fail(WBMM_E_INVALID, "grid offset (%d, %d) outside [0, w=%d)", oy, ox, w);
  const wbmm_status sm = check_map(B, C, H + oy, W + ox, w, layout);
  if (sm != WBMM_OK) return sm;
  wbmm::FwdRequest r = make_fwd(B, C, H, W, w, layout, in_dtype, out_dtype, x, T, M, mix_w, z_save,
                                y, workspace, workspace_bytes);
  r.oy = oy;
  r.ox = ox;
  wbmm_status st = check_forward(r, in_dtype, out_dtype);
  if (st != WBMM_OK) return st;
  const size_t need = wbmm::forward_workspace(r);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(WBMM_E_WORKSPACE, "workspace of %zu bytes required, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (need > 0 && !aligned(workspace, 16))
    return fail(WBMM_E_UNSUPPORTED, "workspace not 16-byte aligned");
  return hip_status(wbmm::launch_forward(r, (hipStream_t)stream), name);
}

}  // namespace

WBMM_API size_t wbmm_forward_workspace_bytes(int B, int C, int H, int W, int w, int layout,
                                             int has_mix, int has_z_save) {
  return forward_ws_bytes(B, C, H, W, w, 0, 0, layout, has_mix, has_z_save);
}

WBMM_API wbmm_status wbmm_forward(int B, int C, int H, int W, int w, int layout, int in_dtype,
                                  int out_dtype, const void* x, const void* T, const void* M,
                                  const float* mix_w, void* z_save, void* y, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return forward_call(B, C, H, W, w, 0, 0, layout, in_dtype, out_dtype, x, T, M, mix_w, z_save, y,
                      workspace, workspace_bytes, stream, "wbmm_forward");
}

WBMM_API size_t wbmm_forward_shifted_workspace_bytes(int B, int C, int H, int W, int w, int oy,
                                                     int ox, int layout, int has_mix,
                                                     int has_z_save) {
  return forward_ws_bytes(B, C, H, W, w, oy, ox, layout, has_mix, has_z_save);
}

WBMM_API wbmm_status wbmm_forward_shifted(int B, int C, int H, int W, int w, int oy, int ox,
                                          int layout, int in_dtype, int out_dtype, const void* x,
                                          const void* T, const void* M, const float* mix_w,
                                          void* z_save, void* y, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  return forward_call(B, C, H, W, w, oy, ox, layout, in_dtype, out_dtype, x, T, M, mix_w, z_save,
                      y, workspace, workspace_bytes, stream, "wbmm_forward_shifted");
}

namespace {

wbmm::BwdRequest make_bwd(int B, int C, int H, int W, int w, int layout, const float* x,
                          const float* T, const float* M, const float* mix_w, const float* z_saved,
                          const float* dy, float* dx, float* dT, float* dmix_w, void* ws,
                          size_t ws_bytes) {
  wbmm::BwdRequest r{};
  r.B = B; r.C = C; r.H = H; r.W = W; r.w = w; r.layout = layout;
  r.x = x; r.T = T; r.M = M; r.mixw = mix_w; r.zsaved = z_saved; r.dy = dy;
  r.dx = dx; r.dT = dT; r.dmixw = mix_w ? dmix_w : nullptr;
  r.ws = ws; r.ws_bytes = ws_bytes;
  return r;
}

}  // namespace

namespace {

size_t backward_ws_bytes(int B, int C, int H, int W, int w, int oy, int ox, int layout,
                         int has_mix) {
  if (check_map(B, C, H + oy, W + ox, w, layout) != WBMM_OK || !offsets_ok(w, oy, ox)) return 0;
  static const float dummy = 0.f;
  wbmm::BwdRequest r = make_bwd(B, C, H, W, w, layout, &dummy, &dummy, nullptr,
                                has_mix ? &dummy : nullptr, has_mix ? &dummy : nullptr, &dummy,
                                nullptr, nullptr, nullptr, nullptr, 0);
  r.oy = oy;
  r.ox = ox;
  if (!wbmm::backward_plan_ok(r)) return 0;
  // the operand kind is not an argument: the larger need of a table and a cached matrix
  size_t need = wbmm::backward_workspace(r);
  r.T = nullptr;
  r.M = &dummy;
  if (wbmm::backward_plan_ok(r)) {
    const size_t n = wbmm::backward_workspace(r);
    if (n > need) need = n;
  }
  return need;
}

}  // namespace

// Scratch of the allocation-free backward: one copy per GPU, in the library's code object, held
// until the process ends. Host code never passes `scratch` itself to a kernel (on the host it is
// only a stand-in for the symbol); it asks for the device address once per device.
static __device__ __align__(256) unsigned char scratch[WBMM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kScratchBytes = WBMM_NOALLOC_SCRATCH_BYTES;
std::mutex g_scratch_mu;
void* g_scratch_dev[64];  // device address of `scratch` per device id, once looked up

// The current device's copy of `scratch` (looked up on first use with that device current).
wbmm_status scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(WBMM_E_UNSUPPORTED, "device id %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(WBMM_E_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return WBMM_OK;
}

// no_alloc: the workspace is the current device's `scratch` (workspace arguments ignored).
wbmm_status backward_call(int B, int C, int H, int W, int w, int oy, int ox, int layout,
                          const float* x, const float* T, const float* M, const float* mix_w,
                          const float* z_saved, const float* dy, float* dx, float* dT,
                          float* dmix_w, void* workspace, size_t workspace_bytes, void* stream,
                          const char* name, bool no_alloc = false) {
  if (!offsets_ok(w, oy, ox))
    return fail(WBMM_E_INVALID, "grid offset (%d, %d) outside [0, w=%d)", oy, ox, w);
  wbmm_status st = check_map(B, C, H + oy, W + ox, w, layout);
  if (st != WBMM_OK) return st;
  if (!x || !dy) return fail(WBMM_E_INVALID, "x and dy must be non-NULL");
  if ((T == nullptr) == (M == nullptr))
    return fail(WBMM_E_INVALID, "exactly one of T (table) and M (cached matrix) must be given");
  if ((mix_w == nullptr) != (z_saved == nullptr))
    return fail(WBMM_E_INVALID, "z_saved is required exactly when mix_w is given");
  const void* ptrs[] = {x, T, M, mix_w, z_saved, dy, dx, dT, dmix_w};
  for (const void* p : ptrs)
    if (p && !aligned(p, 4)) return fail(WBMM_E_UNSUPPORTED, "pointer not 4-byte aligned");
  const size_t mb = (size_t)B * C * H * W * 4;
  const size_t tb = (size_t)C * (2 * w - 1) * (2 * w - 1) * 4;
  if (dx && (overlaps(dx, mb, x, mb) || overlaps(dx, mb, dy, mb) || overlaps(dx, mb, z_saved, mb)))
    return fail(WBMM_E_INVALID, "dx overlaps an input");
  if (dT && (overlaps(dT, tb, T, tb) || overlaps(dT, tb, dx, mb)))
    return fail(WBMM_E_INVALID, "dT overlaps T or dx");
  wbmm::BwdRequest r = make_bwd(B, C, H, W, w, layout, x, T, M, mix_w, z_saved, dy, dx, dT, dmix_w,
                                workspace, workspace_bytes);
  r.oy = oy;
  r.ox = ox;
  if (!wbmm::backward_plan_ok(r))
    return fail(WBMM_E_UNSUPPORTED, "no launch shape fits this problem (w=%d)", w);
  const size_t need = wbmm::backward_workspace(r);
  if (no_alloc) {
    if (need > kScratchBytes)
      return fail(WBMM_E_UNSUPPORTED,
                  "this problem needs %zu bytes of scratch; the allocation-free backward holds "
                  "%zu (use wbmm_backward with a workspace)", need, kScratchBytes);
    const wbmm_status sp = scratch_ptr(&r.ws);
    if (sp != WBMM_OK) return sp;
    r.ws_bytes = kScratchBytes;
    return hip_status(wbmm::launch_backward(r, (hipStream_t)stream), name);
  }
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(WBMM_E_WORKSPACE, "workspace of %zu bytes required, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (need > 0 && !aligned(workspace, 256))
    return fail(WBMM_E_UNSUPPORTED, "workspace not 256-byte aligned");
  return hip_status(wbmm::launch_backward(r, (hipStream_t)stream), name);
}

}  // namespace

WBMM_API size_t wbmm_backward_workspace_bytes(int B, int C, int H, int W, int w, int layout,
                                              int has_mix) {
  return backward_ws_bytes(B, C, H, W, w, 0, 0, layout, has_mix);
}

WBMM_API wbmm_status wbmm_backward(int B, int C, int H, int W, int w, int layout, const float* x,
                                   const float* T, const float* M, const float* mix_w,
                                   const float* z_saved, const float* dy, float* dx, float* dT,
                                   float* dmix_w, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  return backward_call(B, C, H, W, w, 0, 0, layout, x, T, M, mix_w, z_saved, dy, dx, dT, dmix_w,
                       workspace, workspace_bytes, stream, "wbmm_backward");
}

WBMM_API wbmm_status wbmm_backward_noalloc(int B, int C, int H, int W, int w, int layout,
                                           const float* x, const float* T, const float* M,
                                           const float* mix_w, const float* z_saved,
                                           const float* dy, float* dx, float* dT, float* dmix_w,
                                           void* stream) {
  return backward_call(B, C, H, W, w, 0, 0, layout, x, T, M, mix_w, z_saved, dy, dx, dT, dmix_w,
                       nullptr, 0, stream, "wbmm_backward_noalloc", true);
}

WBMM_API size_t wbmm_backward_shifted_workspace_bytes(int B, int C, int H, int W, int w, int oy,
                                                      int ox, int layout, int has_mix) {
  return backward_ws_bytes(B, C, H, W, w, oy, ox, layout, has_mix);
}

WBMM_API wbmm_status wbmm_backward_shifted(int B, int C, int H, int W, int w, int oy, int ox,
                                           int layout, const float* x, const float* T,
                                           const float* M, const float* mix_w,
                                           const float* z_saved, const float* dy, float* dx,
                                           float* dT, float* dmix_w, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  return backward_call(B, C, H, W, w, oy, ox, layout, x, T, M, mix_w, z_saved, dy, dx, dT, dmix_w,
                       workspace, workspace_bytes, stream, "wbmm_backward_shifted");
}
namespace {
// Shared checks of the hierarchical entry points: fp32 tables, s x s sub-windows tiling the
// w x w window (s divides w, s < w).
bool hier_sizes_ok(int w, int s) { return s >= 1 && s < w && w % s == 0; }
wbmm_status check_hier(int w, int s, const float* T, const float* T_sub) {
  if (!hier_sizes_ok(w, s))
    return fail(WBMM_E_INVALID, "the sub-window side must divide the window side and be smaller "
                "(w=%d, s=%d)", w, s);
  if (!T || !T_sub) return fail(WBMM_E_INVALID, "T and T_sub must be non-NULL");
  if (!aligned(T, 4) || !aligned(T_sub, 4)) return fail(WBMM_E_UNSUPPORTED, "misaligned pointer");
  return WBMM_OK;
}
}  // namespace
WBMM_API size_t wbmm_forward_hier_workspace_bytes(int B, int C, int H, int W, int w, int s,
                                                  int layout, int has_mix, int has_z_save) {
  if (check_map(B, C, H, W, w, layout) != WBMM_OK || !hier_sizes_ok(w, s)) return 0;
  static const float dummy = 0.f;
  wbmm::FwdRequest r = make_fwd(B, C, H, W, w, layout, WBMM_F32, WBMM_F32, &dummy, &dummy, nullptr,
                                has_mix ? &dummy : nullptr, has_z_save ? (void*)&dummy : nullptr,
                                (void*)&dummy, nullptr, 0);
  r.Tsub = &dummy;
  r.s = s;
  if (!wbmm::forward_plan_ok(r)) return 0;
  return wbmm::forward_workspace(r);
}
WBMM_API wbmm_status wbmm_forward_hier(int B, int C, int H, int W, int w, int s, int layout,
                                       const float* x, const float* T, const float* T_sub,
                                       const float* mix_w, float* z_save, float* y,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  wbmm_status st = check_map(B, C, H, W, w, layout);
  if (st != WBMM_OK) return st;
  st = check_hier(w, s, T, T_sub);
  if (st != WBMM_OK) return st;
  wbmm::FwdRequest r = make_fwd(B, C, H, W, w, layout, WBMM_F32, WBMM_F32, x, T, nullptr, mix_w,
                                z_save, y, workspace, workspace_bytes);
  r.Tsub = T_sub;
  r.s = s;
  st = check_forward(r, WBMM_F32, WBMM_F32);
  if (st != WBMM_OK) return st;
  const size_t elems = (size_t)B * C * H * W;
  if (overlaps(y, elems * 4, T_sub, (size_t)C * (2 * s - 1) * (2 * s - 1) * 4))
    return fail(WBMM_E_INVALID, "y overlaps T_sub");
  const size_t need = wbmm::forward_workspace(r);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(WBMM_E_WORKSPACE, "workspace of %zu bytes required, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (need > 0 && !aligned(workspace, 16))
    return fail(WBMM_E_UNSUPPORTED, "workspace not 16-byte aligned");
  return hip_status(wbmm::launch_forward(r, (hipStream_t)stream), "wbmm_forward_hier");
}
WBMM_API size_t wbmm_backward_hier_workspace_bytes(int B, int C, int H, int W, int w, int s,
                                                   int layout, int has_mix) {
  if (check_map(B, C, H, W, w, layout) != WBMM_OK || !hier_sizes_ok(w, s)) return 0;
  static const float dummy = 0.f;
  wbmm::BwdRequest r = make_bwd(B, C, H, W, w, layout, &dummy, &dummy, nullptr,
                                has_mix ? &dummy : nullptr, has_mix ? &dummy : nullptr, &dummy,
                                nullptr, nullptr, nullptr, nullptr, 0);
  r.Tsub = &dummy;
  r.s = s;
  if (!wbmm::backward_plan_ok(r)) return 0;
  return wbmm::backward_workspace(r);
}
WBMM_API wbmm_status wbmm_backward_hier(int B, int C, int H, int W, int w, int s, int layout,
                                        const float* x, const float* T, const float* T_sub,
                                        const float* mix_w, const float* z_saved, const float* dy,
                                        float* dx, float* dT, float* dT_sub, float* dmix_w,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  wbmm_status st = check_map(B, C, H, W, w, layout);
  if (st != WBMM_OK) return st;
  st = check_hier(w, s, T, T_sub);
  if (st != WBMM_OK) return st;
  if (!x || !dy) return fail(WBMM_E_INVALID, "x and dy must be non-NULL");
  if ((mix_w == nullptr) != (z_saved == nullptr))
    return fail(WBMM_E_INVALID, "z_saved is required exactly when mix_w is given");
  const void* ptrs[] = {x, mix_w, z_saved, dy, dx, dT, dT_sub, dmix_w};
  for (const void* p : ptrs)
    if (p && !aligned(p, 4)) return fail(WBMM_E_UNSUPPORTED, "pointer not 4-byte aligned");
  const size_t mb = (size_t)B * C * H * W * 4;
  const size_t tb = (size_t)C * (2 * w - 1) * (2 * w - 1) * 4;
  const size_t sb = (size_t)C * (2 * s - 1) * (2 * s - 1) * 4;
  if (dx && (overlaps(dx, mb, x, mb) || overlaps(dx, mb, dy, mb) || overlaps(dx, mb, z_saved, mb)))
    return fail(WBMM_E_INVALID, "dx overlaps an input");
  if (dT && (overlaps(dT, tb, T, tb) || overlaps(dT, tb, T_sub, sb) || overlaps(dT, tb, dx, mb)))
    return fail(WBMM_E_INVALID, "dT overlaps T, T_sub or dx");
  if (dT_sub && (overlaps(dT_sub, sb, T, tb) || overlaps(dT_sub, sb, T_sub, sb) ||
                 overlaps(dT_sub, sb, dx, mb) || overlaps(dT_sub, sb, dT, tb)))
    return fail(WBMM_E_INVALID, "dT_sub overlaps T, T_sub, dx or dT");
  wbmm::BwdRequest r = make_bwd(B, C, H, W, w, layout, x, T, nullptr, mix_w, z_saved, dy, dx, dT,
                                dmix_w, workspace, workspace_bytes);
  r.Tsub = T_sub;
  r.s = s;
  r.dTsub = dT_sub;
  if (!wbmm::backward_plan_ok(r))
    return fail(WBMM_E_UNSUPPORTED, "no launch shape fits this problem (w=%d)", w);
  const size_t need = wbmm::backward_workspace(r);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(WBMM_E_WORKSPACE, "workspace of %zu bytes required, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (need > 0 && !aligned(workspace, 256))
    return fail(WBMM_E_UNSUPPORTED, "workspace not 256-byte aligned");
  return hip_status(wbmm::launch_backward(r, (hipStream_t)stream), "wbmm_backward_hier");
}

WBMM_API wbmm_status wbmm_dwconv_forward(int B, int C, int H, int W, int k, const float* x,
                                         const float* w_dw, float* y, void* stream) {
  if (B < 1 || C < 1 || H < 1 || W < 1)
    return fail(WBMM_E_INVALID, "sizes must be >= 1 (B=%d C=%d H=%d W=%d)", B, C, H, W);
  if (k < 1 || k % 2 == 0) return fail(WBMM_E_INVALID, "kernel size k=%d must be odd and >= 1", k);
  if (!x || !w_dw || !y) return fail(WBMM_E_INVALID, "x, w_dw and y must be non-NULL");
  if (!aligned(x, 4) || !aligned(w_dw, 4) || !aligned(y, 4))
    return fail(WBMM_E_UNSUPPORTED, "pointer not 4-byte aligned");
  if (!wbmm::dwconv_supported(B, C, H, W, k))
    return fail(WBMM_E_UNSUPPORTED,
                "the depthwise convolution is provided for odd k in 3..13 and rows up to ~600 "
                "pixels (k=%d, W=%d)", k, W);
  const size_t mb = (size_t)B * C * H * W * 4;
  if (overlaps(y, mb, x, mb)) return fail(WBMM_E_INVALID, "y overlaps x");
  if (overlaps(y, mb, w_dw, (size_t)C * k * k * 4)) return fail(WBMM_E_INVALID, "y overlaps w_dw");
  return hip_status(wbmm::launch_dwconv(B, C, H, W, k, x, w_dw, y, (hipStream_t)stream),
                    "wbmm_dwconv_forward");
}

WBMM_API double wbmm_probe_mfma_flops(int dtype, int blocks, int iters) {
  if (!valid_dtype(dtype) || blocks < 1 || iters < 1) return 0.0;
  return wbmm::probe_mfma_flops(dtype == WBMM_BF16, blocks, iters);
}

WBMM_API wbmm_status wbmm_probe_mfma(int dtype, int blocks, int iters, float* out, void* stream) {
  if (!valid_dtype(dtype)) return fail(WBMM_E_INVALID, "unknown dtype %d", dtype);
  if (blocks < 1 || iters < 1 || blocks > 1 << 20)
    return fail(WBMM_E_INVALID, "blocks=%d and iters=%d must be >= 1 (blocks <= 2^20)", blocks,
                iters);
  if (!out || !aligned(out, 4)) return fail(WBMM_E_INVALID, "out must be a 4-byte aligned pointer");
  return hip_status(wbmm::launch_probe_mfma(dtype == WBMM_BF16, blocks, iters, out,
                                            (hipStream_t)stream),
                    "wbmm_probe_mfma");
}

WBMM_API size_t wbmm_backward_bf16_workspace_bytes(int B, int C, int H, int W, int w, int layout,
                                                   int has_mix) {
  if (check_map(B, C, H, W, w, layout) != WBMM_OK ||
      !wbmm::bf16_backward_plan_ok(B, C, H, W, w, layout))
    return 0;
  return wbmm::bf16_backward_workspace(B, C, H, W, w, layout, has_mix);
}

WBMM_API wbmm_status wbmm_backward_bf16(int B, int C, int H, int W, int w, int layout,
                                        const void* x, const void* T, const float* mix_w,
                                        const void* z_saved, const void* dy, void* dx, float* dT,
                                        float* dmix_w, void* workspace, size_t workspace_bytes,
                                        void* stream) {
  wbmm_status st = check_map(B, C, H, W, w, layout);
  if (st != WBMM_OK) return st;
  if (!wbmm::bf16_backward_plan_ok(B, C, H, W, w, layout))
    return fail(WBMM_E_UNSUPPORTED, "no launch shape fits this problem (w=%d)", w);
  if (!x || !T || !dy) return fail(WBMM_E_INVALID, "x, T and dy must be non-NULL");
  if ((mix_w == nullptr) != (z_saved == nullptr))
    return fail(WBMM_E_INVALID, "z_saved is required exactly when mix_w is given");
  const void* ptrs[] = {x, T, z_saved, dy, dx};
  for (const void* p : ptrs)
    if (p && !aligned(p, 16)) return fail(WBMM_E_UNSUPPORTED, "bf16 maps and T must be 16-byte aligned");
  const void* fptrs[] = {mix_w, dT, dmix_w};
  for (const void* p : fptrs)
    if (p && !aligned(p, 4)) return fail(WBMM_E_UNSUPPORTED, "pointer not 4-byte aligned");
  const size_t mb = (size_t)B * C * H * W * 2;
  const size_t tb = (size_t)C * (2 * w - 1) * (2 * w - 1);
  if (dx && (overlaps(dx, mb, x, mb) || overlaps(dx, mb, dy, mb) || overlaps(dx, mb, z_saved, mb) ||
             overlaps(dx, mb, T, tb * 2)))
    return fail(WBMM_E_INVALID, "dx overlaps an input");
  if (dT && (overlaps(dT, tb * 4, T, tb * 2) || overlaps(dT, tb * 4, dx, mb)))
    return fail(WBMM_E_INVALID, "dT overlaps T or dx");
  if (dmix_w && mix_w && overlaps(dmix_w, (size_t)C * 36, mix_w, (size_t)C * 36))
    return fail(WBMM_E_INVALID, "dmix_w overlaps mix_w");
  const size_t need = wbmm::bf16_backward_workspace(B, C, H, W, w, layout, mix_w != nullptr);
  if (!workspace || workspace_bytes < need)
    return fail(WBMM_E_WORKSPACE, "workspace of %zu bytes required, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 256)) return fail(WBMM_E_UNSUPPORTED, "workspace not 256-byte aligned");
  wbmm::BwdBf16Request r{};
  r.B = B; r.C = C; r.H = H; r.W = W; r.w = w; r.layout = layout;
  r.x = (const uint16_t*)x; r.T = (const uint16_t*)T; r.mixw = mix_w;
  r.zsaved = (const uint16_t*)z_saved; r.dy = (const uint16_t*)dy; r.dx = (uint16_t*)dx;
  r.dT = dT; r.dmixw = mix_w ? dmix_w : nullptr; r.ws = workspace;
  return hip_status(wbmm::launch_backward_bf16(r, (hipStream_t)stream), "wbmm_backward_bf16");
}
