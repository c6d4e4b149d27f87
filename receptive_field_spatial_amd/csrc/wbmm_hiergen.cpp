// The layer with an s x s sub-window table folded in, for sub-windows other than the window's
// quadrants (s divides w, s < w, w != 2s) and for w = 2s above 16 (w = 2s <= 16 folds on chip
// in the fast and general kernels). The fold adds T_sub_c[(dy, dx) + s - 1] to M_c[i][j] for
// the pairs i, j of one s x s sub-window [gecl.asia reading notes, "Method": the 7 x 7 table
// folded into the 14 x 14 matrix, here for any s | w]. Host orchestration of existing kernels:
//   forward:  M' = fold(M(T), T_sub) built in the workspace, then the cached-matrix forward;
//   backward: M' as above; G = mix adjoint of dy (with the dWmix sums) when there is a mix;
//             dX and dT from the cached-matrix backward on G; dT_sub as the table gradient of an
//             s-window layer on the same G and x: a pair of one sub-window with offset d is a
//             pair of one window of the s-grid (which the w-grid subdivides) with offset d, and
//             padding pixels are zero in both grids.
#include "wbmm_launch.hpp"

namespace wbmm {

namespace {

size_t al256(size_t v) { return (v + 255) / 256 * 256; }

size_t folded_bytes(int C, int w) { return al256((size_t)C * w * w * w * w * sizeof(float)); }

FwdRequest cached_fwd(const FwdRequest& r, const float* Mf) {
  FwdRequest q = r;
  q.T = nullptr;
  q.M = Mf;
  q.Tsub = nullptr;
  q.s = 0;
  return q;
}

// [M' (C d^2 floats)] [G map (mix)] [dWmix partials (mix, NCHW planes pass)] [sub-call workspace]
struct HierBwdWs {
  size_t gmap, partW, sub, total;
};

HierBwdWs hier_bwd_ws(const BwdRequest& r, const BwdRequest& main_q, const BwdRequest& sub_q) {
  const bool mix = r.mixw != nullptr;
  const bool pass = mix && r.layout == 0 && mix_bwd_pass_ok(r.H, r.W);
  HierBwdWs w{};
  w.gmap = folded_bytes(r.C, r.w);
  w.partW = w.gmap + (mix ? al256((size_t)r.B * r.C * r.H * r.W * sizeof(float)) : 0);
  w.sub = w.partW + (pass ? al256((size_t)r.C * mix_bwd_parts(r.B, r.H, r.W) * 9 * 8) : 0);
  const size_t a = backward_workspace(main_q), b = r.dTsub ? backward_workspace(sub_q) : 0;
  w.total = w.sub + (a > b ? a : b);
  return w;
}

// The two backward calls of the composition (pointers into the workspace filled in at launch).
void hier_bwd_requests(const BwdRequest& r, const float* Mf, const float* gmap, BwdRequest& main_q,
                       BwdRequest& sub_q) {
  main_q = r;
  main_q.T = nullptr;
  main_q.M = Mf;
  main_q.Tsub = nullptr;
  main_q.s = 0;
  main_q.dTsub = nullptr;
  main_q.mixw = nullptr;
  main_q.zsaved = nullptr;
  main_q.dmixw = nullptr;
  main_q.dy = gmap;
  sub_q = main_q;
  sub_q.w = r.s;
  sub_q.M = nullptr;
  sub_q.T = r.Tsub;  // the table of an s-window layer; only its gradient is asked for
  sub_q.dx = nullptr;
  sub_q.dT = r.dTsub;
}

}  // namespace

// The on-chip fold covers w = 2s up to w = 16; everything else with a sub-table comes here.
bool hier_general(const FwdRequest& r) { return r.Tsub && (2 * r.s != r.w || r.w > 16); }
bool hier_general(const BwdRequest& r) { return r.Tsub && (2 * r.s != r.w || r.w > 16); }

bool hier_forward_plan_ok(const FwdRequest& r) {
  static const float dummy = 0.f;
  return r.s >= 1 && r.s < r.w && r.w % r.s == 0 && !r.in_bf16 && !r.out_bf16 &&
         forward_plan_ok(cached_fwd(r, &dummy));
}

size_t hier_forward_workspace(const FwdRequest& r) {
  static const float dummy = 0.f;
  return folded_bytes(r.C, r.w) + forward_workspace(cached_fwd(r, &dummy));
}

hipError_t launch_forward_hier_general(const FwdRequest& r, hipStream_t st) {
  if (!hier_forward_plan_ok(r)) return hipErrorInvalidValue;
  unsigned char* ws = (unsigned char*)r.ws;
  float* Mf = (float*)ws;
  hipError_t e = launch_build_matrix(r.T, r.C, r.w, 0, Mf, st);
  if (e != hipSuccess) return e;
  e = launch_fold(Mf, r.Tsub, r.C, r.w, r.s, 0, Mf, st);  // in place
  if (e != hipSuccess) return e;
  FwdRequest q = cached_fwd(r, Mf);
  const size_t off = folded_bytes(r.C, r.w);
  q.ws = ws + off;
  q.ws_bytes = r.ws_bytes > off ? r.ws_bytes - off : 0;
  return launch_forward(q, st);
}

bool hier_backward_plan_ok(const BwdRequest& r) {
  if (r.s < 1 || r.s >= r.w || r.w % r.s != 0) return false;
  static const float dummy = 0.f;
  BwdRequest main_q, sub_q;
  hier_bwd_requests(r, &dummy, &dummy, main_q, sub_q);
  return backward_plan_ok(main_q) && (!r.dTsub || backward_plan_ok(sub_q));
}

size_t hier_backward_workspace(const BwdRequest& r) {
  static const float dummy = 0.f;
  BwdRequest main_q, sub_q;
  hier_bwd_requests(r, &dummy, &dummy, main_q, sub_q);
  return hier_bwd_ws(r, main_q, sub_q).total;
}

hipError_t launch_backward_hier_general(const BwdRequest& r, hipStream_t st) {
  if (!hier_backward_plan_ok(r)) return hipErrorInvalidValue;
  unsigned char* ws = (unsigned char*)r.ws;
  float* Mf = (float*)ws;
  const bool mix = r.mixw != nullptr;
  BwdRequest main_q, sub_q;
  hier_bwd_requests(r, Mf, r.dy, main_q, sub_q);  // with a mix, dy becomes G below
  const HierBwdWs wl = hier_bwd_ws(r, main_q, sub_q);
  float* gm = mix ? (float*)(ws + wl.gmap) : nullptr;
  hipError_t e = launch_build_matrix(r.T, r.C, r.w, 0, Mf, st);
  if (e != hipSuccess) return e;
  e = launch_fold(Mf, r.Tsub, r.C, r.w, r.s, 0, Mf, st);  // in place
  if (e != hipSuccess) return e;
  if (mix) {  // G (and dWmix) on the whole map
    if (r.layout == 0 && mix_bwd_pass_ok(r.H, r.W)) {
      double* partW = (double*)(ws + wl.partW);
      e = launch_mix_bwd_planes_f32(r.dy, r.dmixw ? r.zsaved : nullptr, r.mixw, gm, partW, r.B,
                                    r.C, r.H, r.W, st);
      if (e != hipSuccess) return e;
      if (r.dmixw) {
        e = launch_bwd_reduce2(nullptr, 0, partW, mix_bwd_parts(r.B, r.H, r.W), r.C, 0, nullptr,
                               r.dmixw, st);
        if (e != hipSuccess) return e;
      }
    } else {
      e = launch_mix_bwd_data_t<float>(r.dy, r.mixw, gm, r.B, r.C, r.H, r.W, r.layout, st);
      if (e != hipSuccess) return e;
      if (r.dmixw) {
        e = launch_mix_bwd_weight_t<float>(r.dy, r.zsaved, r.dmixw, r.B, r.C, r.H, r.W, r.layout,
                                           st);
        if (e != hipSuccess) return e;
      }
    }
    main_q.dy = gm;
    sub_q.dy = gm;
  }
  main_q.ws = ws + wl.sub;
  main_q.ws_bytes = wl.total - wl.sub;
  sub_q.ws = ws + wl.sub;
  sub_q.ws_bytes = wl.total - wl.sub;
  if (r.dx || r.dT) {
    e = launch_backward(main_q, st);
    if (e != hipSuccess) return e;
  }
  if (r.dTsub) return launch_backward(sub_q, st);
  return hipSuccess;
}

}  // namespace wbmm
