// Host-side launch interface between the C ABI (wbmm_api.cpp) and the kernel translation units.
// Everything here assumes arguments already validated by the API layer.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace wbmm {

struct FwdRequest {
  int B, C, H, W, w, layout, in_bf16, out_bf16;
  const void* x;
  const void* T;  // exactly one of T / M
  const void* M;
  const float* mixw;
  void* zsave;
  void* y;
  void* ws;
  size_t ws_bytes;
  const float* Tsub;  // s x s sub-window tables folded on chip (fp32 table path, w = 2s), or null
  int s;
  int oy, ox;         // window grid offset (0 <= oy, ox < w); the fast paths take 0, 0 only
  int flip;           // contract with M^T (fp32 cached matrix, no mix; the backward's dX)
};

struct BwdRequest {
  int B, C, H, W, w, layout;
  const float* x;
  const float* T;
  const float* M;
  const float* mixw;
  const float* zsaved;
  const float* dy;
  float* dx;
  float* dT;
  float* dmixw;
  void* ws;
  size_t ws_bytes;
  const float* Tsub;  // as in FwdRequest; with it, dTsub (or null) receives the sub-table gradient
  int s;
  float* dTsub;
  int oy, ox;         // as in FwdRequest
};

hipError_t launch_build_index(int w, int32_t* idx, hipStream_t st);
hipError_t launch_build_matrix(const void* T, int C, int w, int bf16, void* M, hipStream_t st);
hipError_t launch_fold(const void* Min, const void* Tsub, int C, int w, int s, int bf16,
                       void* Mout, hipStream_t st);

// Returns false when no launch shape exists (reported as unsupported by the caller).
bool forward_plan_ok(const FwdRequest& r);
size_t forward_workspace(const FwdRequest& r);
hipError_t launch_forward(const FwdRequest& r, hipStream_t st);
// The hierarchical layer for sub-windows other than the quadrants, or w = 2s > 16 (Tsub set,
// s | w, s < w): the folded matrix built in the workspace, then the cached-matrix kernels (and for
// the backward the s-window table gradient as dT_sub).
bool hier_general(const FwdRequest& r);
bool hier_general(const BwdRequest& r);
bool hier_forward_plan_ok(const FwdRequest& r);
size_t hier_forward_workspace(const FwdRequest& r);
hipError_t launch_forward_hier_general(const FwdRequest& r, hipStream_t st);
bool hier_backward_plan_ok(const BwdRequest& r);
size_t hier_backward_workspace(const BwdRequest& r);
hipError_t launch_backward_hier_general(const BwdRequest& r, hipStream_t st);
// Backward for 16 < w <= 32 (fp32 or bf16 maps: map_bytes 4 or 2; the request's map and table
// pointers point at data of that type).
bool wide_backward_ok(const BwdRequest& r);
size_t backward_wide_workspace(const BwdRequest& r, size_t map_bytes);
hipError_t launch_backward_wide(const BwdRequest& r, bool bf16, hipStream_t st);

bool backward_plan_ok(const BwdRequest& r);
size_t backward_workspace(const BwdRequest& r);
hipError_t launch_backward(const BwdRequest& r, hipStream_t st);

// Fast fp32 paths for w = 14, NCHW, square images of 14, 28 or 56 (whole images per wave).
bool fast_forward_ok(const FwdRequest& r);
hipError_t launch_forward_fast(const FwdRequest& r, hipStream_t st);
bool fast_backward_ok(const BwdRequest& r);
size_t fast_backward_workspace(const BwdRequest& r);
hipError_t launch_backward_fast(const BwdRequest& r, hipStream_t st);
// Per-image element offsets of the fast kernels stay in 32 bits.
bool offsets_fit(int C, int H, int W);

// Offset window grids (w = 14, NCHW, table input, no sub-table; fp32 maps, or bf16 maps without
// the mix in the forward) on the fast kernels: the grid's windows are gathered into whole 28x28
// images in the workspace and the results put back.
bool fast_roll_forward_ok(const FwdRequest& r);
size_t fast_roll_forward_workspace(const FwdRequest& r);
hipError_t launch_forward_fast_roll(const FwdRequest& r, hipStream_t st);
bool fast_roll_backward_ok(const BwdRequest& r);
size_t fast_roll_backward_workspace(const BwdRequest& r);
hipError_t launch_backward_fast_roll(const BwdRequest& r, hipStream_t st);
bool roll_backward_ok(const BwdRequest& r);
size_t roll_backward_workspace(const BwdRequest& r);
hipError_t launch_backward_rolled(const BwdRequest& r, hipStream_t st);
bool repack_forward_ok(const FwdRequest& r);
size_t repack_forward_workspace(const FwdRequest& r);
hipError_t launch_forward_repacked(const FwdRequest& r, hipStream_t st);
bool repack_backward_ok(const BwdRequest& r);
size_t repack_backward_workspace(const BwdRequest& r);
hipError_t launch_backward_repacked(const BwdRequest& r, hipStream_t st);

// Fast fp32 forward on a cached matrix (w = 14, NCHW, any H and W, no sub-table, plain grid):
// the contraction's result goes to `out` (and a copy to `out2` when not null).
bool fast_cm_forward_ok(const FwdRequest& r);
// Fast fp32 forward from the table (w = 14, NCHW, any H and W, plain grid; a 7 x 7 sub-table
// folded on chip when Tsub is set): the contraction into out (and out2 when not null).
bool fast_tab_forward_ok(const FwdRequest& r);
hipError_t launch_forward_fast_tab(const FwdRequest& r, float* out, float* out2, hipStream_t st);
// fp32 w = 7 and w = 28 on NCHW 56x56 maps, table input: the contraction into out (and out2
// when not null).
bool fast_f32_w7_forward_ok(const FwdRequest& r);
hipError_t launch_forward_fast_f32_w7(const FwdRequest& r, float* out, float* out2,
                                      hipStream_t st);
bool fast_f32_w28_forward_ok(const FwdRequest& r);
hipError_t launch_forward_fast_f32_w28(const FwdRequest& r, float* out, float* out2,
                                       hipStream_t st);
hipError_t launch_forward_fast_cm(const FwdRequest& r, float* out, float* out2, hipStream_t st);

// Fast bf16 forwards for NCHW table input, bf16 output, no mix: w = 14 on 28x28 and 56x56
// images, w = 7 and w = 28 on 56x56 images.
bool fast_bf16_forward_ok(const FwdRequest& r);
hipError_t launch_forward_fast_bf16(const FwdRequest& r, hipStream_t st);
// The same w = 14 kernel with the 3x3 mix fused (bf16 y and z_save).
bool fast_bf16_fused_mix_ok(const FwdRequest& r);
hipError_t launch_forward_fast_bf16_mix(const FwdRequest& r, hipStream_t st);

// Fixed-order sum of per-workgroup fp64 partials: dT[c][q] = sum_k partT[c][k][q] (and dWmix).
hipError_t launch_bwd_reduce(const double* partT, const double* partW, int parts, int C, int L,
                             float* dT, float* dmixw, hipStream_t st);
// The same with separate partial counts for dT and dWmix (one launch for both).
hipError_t launch_bwd_reduce2(const double* partT, int partsT, const double* partW, int partsW,
                              int C, int L, float* dT, float* dmixw, hipStream_t st);

// Hands out the caller's timing events (null if none were set for this thread); a pair is used
// by one launch only.
void take_main_events(hipEvent_t* before, hipEvent_t* after);

// Launches a call's main contraction kernel. Timing events armed by the caller are attached to
// the dispatch itself, so they time the kernel's execution rather than the queue around it.
template <class K, class... A>
hipError_t launch_main(K kernel, dim3 grid, dim3 block, unsigned lds, hipStream_t st, A... args) {
  hipEvent_t before = nullptr, after = nullptr;
  take_main_events(&before, &after);
  if (before)
    hipExtLaunchKernelGGL(kernel, grid, block, lds, st, before, after, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, st, args...);
  return hipGetLastError();
}

// bf16 backward (w = 14, NCHW 28x28 / 56x56 images, table input): maps and table in bf16,
// dT and dWmix in fp32.
struct BwdBf16Request {
  int B, C, H, W, w, layout;
  const uint16_t* x;
  const uint16_t* T;
  const float* mixw;
  const uint16_t* zsaved;
  const uint16_t* dy;
  uint16_t* dx;
  float* dT;
  float* dmixw;
  void* ws;
};
bool bf16_backward_ok(int B, int C, int H, int W, int w, int layout);
// The fast bf16 shapes above, or any shape the general kernels plan (w <= 16, any layout).
bool bf16_backward_plan_ok(int B, int C, int H, int W, int w, int layout);
size_t bf16_backward_workspace(int B, int C, int H, int W, int w, int layout, int has_mix);
// bf16 maps and table through the general kernels (fp32 tiles and matrix cores, exact widening;
// the request's map and table pointers point at bf16 data).
size_t backward_bf16_general_workspace(const BwdRequest& r);
hipError_t launch_backward_bf16_general(const BwdRequest& r, hipStream_t st);
hipError_t launch_backward_bf16(const BwdBf16Request& r, hipStream_t st);
hipError_t launch_bf16_transposed_contraction(const uint16_t* g, const uint16_t* T, uint16_t* out,
                                              int B, int C, int H, hipStream_t st);
hipError_t launch_mix_fwd_planes_bf16(const uint16_t* z, const float* w9, uint16_t* y, int B,
                                      int C, int H, int W, hipStream_t st);
// The mix adjoint passes below (G and dWmix partials in one pass over dy and z): planes of even
// width take the direct pass (any size), odd widths the plane-staged one when a plane fits in
// LDS. Their dWmix partials: [C][mix_bwd_parts(B, H, W)][9].
bool mix_bwd_pass_ok(int H, int W);
int mix_bwd_parts(int B, int H, int W);
hipError_t launch_mix_bwd_planes_bf16(const uint16_t* dy, const uint16_t* z, const float* w9,
                                      uint16_t* g, double* partW, int B, int C, int H, int W,
                                      hipStream_t st);
// The same mix passes on fp32 NCHW maps (odd widths need mix_planes_lds_bytes(H, W) and
// (H + 2) (W + 2) 4 bytes per staged plane within 64 KB; they return hipErrorInvalidValue else).
size_t mix_planes_lds_bytes(int H, int W);
// fp32 NCHW forward mix pass: the direct pass for even widths, else the plane-staged pass when a
// plane fits in LDS, else launch_mix_fwd.
hipError_t launch_mix_fwd_f32_route(const float* z, const float* w9, float* y, int B, int C,
                                    int H, int W, hipStream_t st);
hipError_t launch_mix_fwd_planes_f32(const float* z, const float* w9, float* y, int B, int C,
                                     int H, int W, hipStream_t st);
hipError_t launch_mix_bwd_planes_f32(const float* dy, const float* z, const float* w9, float* g,
                                     double* partW, int B, int C, int H, int W, hipStream_t st);

// Matrix-core peak probe (measurement aid): flops of one launch, and the launch.
double probe_mfma_flops(int bf16, int blocks, int iters);
hipError_t launch_probe_mfma(int bf16, int blocks, int iters, float* out, hipStream_t st);

// k x k depthwise convolution (DW-Std), fp32 NCHW, odd k in 3..13.
bool dwconv_supported(int B, int C, int H, int W, int k);
hipError_t launch_dwconv(int B, int C, int H, int W, int k, const float* x, const float* w,
                         float* y, hipStream_t st);

// 3x3 depthwise mix kernels (used by the window-mode paths).
hipError_t launch_mix_fwd(const float* z, const float* w9, void* y, int out_bf16, int B, int C,
                          int H, int W, int layout, hipStream_t st, uint16_t* zcopy = nullptr);
hipError_t launch_mix_bwd_data(const float* dy, const float* w9, float* dz, int B, int C, int H,
                               int W, int layout, hipStream_t st);
hipError_t launch_mix_bwd_weight(const float* dy, const float* z, float* dw9, int B, int C, int H,
                                 int W, int layout, hipStream_t st);
// The same two passes on fp32 or bf16 maps (TM = float or uint16_t; dz in the map type).
template <typename TM>
hipError_t launch_mix_bwd_data_t(const TM* dy, const float* w9, TM* dz, int B, int C, int H,
                                 int W, int layout, hipStream_t st);
template <typename TM>
hipError_t launch_mix_bwd_weight_t(const TM* dy, const TM* z, float* dw9, int B, int C, int H,
                                   int W, int layout, hipStream_t st);

}  // namespace wbmm
