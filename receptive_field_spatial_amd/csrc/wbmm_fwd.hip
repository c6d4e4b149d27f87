// WBMM forward on gfx950: one fused kernel per call in image mode (partition, on-chip M_c,
// MFMA contraction, reverse, optional 3x3 inter-block mix, optional save of the pre-mix map);
// window mode adds a separate mix pass when the mix is requested.
#include "wbmm_core.hpp"
#include "wbmm_launch.hpp"

namespace wbmm {

struct FwdArgs {
  Geo g;
  const void* x;
  const void* tab;
  const void* mat;
  const float* mixw;
  void* zsave;     // pre-mix output, or null
  void* y;         // layer output (window mode with a mix: the pre-mix buffer)
  int out_bf16;
  int mix_here;    // apply the 3x3 mix in this kernel (image mode only)
  const float* tsub;  // sub-window tables folded on chip (HIER), or null
};

// FLIP: contract with M^T instead of M (the backward's dX of a cached matrix, fp32).
template <typename TIn, int RPW, int WR, int ASRC, bool HIER = false, bool FLIP = false>
__global__ void __launch_bounds__(kThreads) k_wbmm_fwd(FwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const Geo& g = a.g;
  constexpr bool kBf16 = sizeof(TIn) == 2;
  const int c = blockIdx.y;
  const int colgrp = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int wr = wave % WR, ct = wave / WR;

  unsigned char* big = smem + g.lds_big;
  const int xtile_bytes = g.NT * (kBf16 ? g.XSB * 2 : g.XR * 4);
  unsigned char* mchunk = big + xtile_bytes;
  unsigned char* tab = smem + g.lds_tab;
  int* offs = (int*)(smem + g.lds_off);

  if constexpr (kBf16) {
    if constexpr (ASRC == 0) load_table_bf16(g, (const uint16_t*)a.tab, c, (uint16_t*)tab, offs);
  } else {
    load_table_f32(g, ASRC == 0 ? (const float*)a.tab : nullptr, c, (float*)tab, (int2*)offs,
                   a.tsub);
  }
  load_xtile<TIn>(g, (const TIn*)a.x, c, colgrp, big);  // ends with a barrier

  v4f acc[RPW];
  if constexpr (kBf16) {
    contract_bf16<RPW, WR, ASRC>(g, c, (const uint16_t*)a.mat, (const uint16_t*)big,
                                 (uint16_t*)mchunk, (const uint16_t*)tab, offs, wr, ct, acc);
  } else {
    contract_f32<RPW, WR, ASRC, FLIP, HIER>(g, c, (const float*)a.mat, (const float*)big,
                                             (float*)mchunk, (const float*)tab, (const int2*)offs,
                                             wr, ct, acc);
  }

  if (!g.image_mode) {
    store_acc_direct<RPW>(g, colgrp, wr, ct, acc, c, a.y, a.zsave, a.out_bf16);
    return;
  }

  // Image mode: stage z as (H+2) x (W+2) planes with a zero halo, then write rows out.
  __syncthreads();  // every wave is done reading the X tile
  float* St = (float*)big;
  const int plane = g.PH * g.PW;
  zero_lds(St, g.ipw * plane);
  __syncthreads();
  stage_acc<RPW>(g, colgrp, wr, ct, acc, St);
  __syncthreads();

  float w9[9];
  if (a.mix_here) {
#pragma unroll
    for (int q = 0; q < 9; ++q) w9[q] = a.mixw[c * 9 + q];
  }
  const int total = g.ipw * g.H * g.W;
  for (int e = threadIdx.x; e < total; e += kThreads) {
    uint32_t img, rem, h, v;
    fdivmod((uint32_t)e, g.fd_HW, img, rem);
    fdivmod(rem, g.fd_W, h, v);
    const int b = colgrp * g.ipw + (int)img;
    if (b >= g.B) continue;
    const float* P = St + (int)img * plane;
    const float z = P[(h + 1) * g.PW + v + 1];
    const size_t off = map_off(g.layout, b, c, (int)h, (int)v, g.C, g.H, g.W);
    if (a.zsave) store_out(a.zsave, off, z, a.out_bf16);
    float yv = z;
    if (a.mix_here) {
      yv = 0.f;
#pragma unroll
      for (int u = 0; u < 3; ++u)
#pragma unroll
        for (int t = 0; t < 3; ++t) yv = fmaf(w9[u * 3 + t], P[(h + u) * g.PW + v + t], yv);
    }
    store_out(a.y, off, yv, a.out_bf16);
  }
}

// ---------------------------------------------------------------------------- dispatch
template <typename TIn, int RPW, int WR, int ASRC, bool HIER = false, bool FLIP = false>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t st) {
  static_assert(!FLIP || sizeof(TIn) == 4, "M^T contraction: fp32 only");
  auto fn = k_wbmm_fwd<TIn, RPW, WR, ASRC, HIER, FLIP>;
  hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     a.g.lds_total);
  if (e != hipSuccess) return e;
  return launch_main(fn, dim3(a.g.col_groups, a.g.C, 1), dim3(kThreads), a.g.lds_total, st, a);
}

template <typename TIn, int ASRC, bool HIER = false, bool FLIP = false>
static hipError_t launch_fwd_tiles(const FwdArgs& a, hipStream_t st) {
  const int RPW = a.g.RPW, WR = a.g.WR;
  if (WR == 1) {
    if (RPW == 4) return launch_fwd_t<TIn, 4, 1, ASRC, HIER, FLIP>(a, st);
    if (RPW == 7) return launch_fwd_t<TIn, 7, 1, ASRC, HIER, FLIP>(a, st);
    if (RPW == 13) return launch_fwd_t<TIn, 13, 1, ASRC, HIER, FLIP>(a, st);
    if (RPW == 16) return launch_fwd_t<TIn, 16, 1, ASRC, HIER, FLIP>(a, st);
  } else {
    if (RPW == 13) return launch_fwd_t<TIn, 13, 4, ASRC, HIER, FLIP>(a, st);
    if (RPW == 16) return launch_fwd_t<TIn, 16, 4, ASRC, HIER, FLIP>(a, st);
  }
  return hipErrorInvalidValue;
}

// Image mode is used when the mix must run in-kernel, or when whole images fill at least three
// quarters of a workgroup's columns.
static bool plan_fwd(Geo& g, const FwdRequest& r) {
  const bool cached = r.M != nullptr;
  const bool mix = r.mixw != nullptr;
  const int s = r.Tsub ? r.s : 0;
  if (!plan_geo(g, r.B, r.C, r.H, r.W, r.w, r.layout, r.in_bf16, cached, true, 0, s, r.oy, r.ox)) {
    if (!plan_geo(g, r.B, r.C, r.H, r.W, r.w, r.layout, r.in_bf16, cached, false, 0, s, r.oy, r.ox)) return false;
  }
  if (g.image_mode && !mix && 4 * g.ipw * g.nWin < 3 * g.NT) {
    if (!plan_geo(g, r.B, r.C, r.H, r.W, r.w, r.layout, r.in_bf16, cached, false, 0, s, r.oy, r.ox)) return false;
  }
  return true;
}

bool forward_plan_ok(const FwdRequest& r) {
  if (hier_general(r)) return hier_forward_plan_ok(r);
  Geo g;
  return plan_fwd(g, r);
}

// bf16 maps with the mix on a fast bf16 shape: the fast forward writes z (bf16) to z_save or the
// workspace, then a plane-staged pass applies the mix (y = bf16(mix(bf16 z))).
static bool fast_bf16_mix_ok(const FwdRequest& r) {
  if (!r.mixw || r.Tsub || !r.in_bf16 || !r.out_bf16 || fast_bf16_fused_mix_ok(r)) return false;
  FwdRequest q = r;
  q.mixw = nullptr;
  q.zsave = nullptr;
  return fast_bf16_forward_ok(q) && (size_t)(r.H + 2) * (r.W + 2) * 4 <= 64 * 1024;
}

size_t forward_workspace(const FwdRequest& r) {
  if (hier_general(r)) return hier_forward_workspace(r);
  if (fast_roll_forward_ok(r)) return fast_roll_forward_workspace(r);
  // the fast kernels that leave the mix to a pass of its own: with the mix, the pre-mix map goes
  // to z_save or here
  if (fast_cm_forward_ok(r) || fast_f32_w28_forward_ok(r) || fast_f32_w7_forward_ok(r) ||
      (!fast_forward_ok(r) && fast_tab_forward_ok(r)))
    return r.mixw && !r.zsave ? (size_t)r.B * r.C * r.H * r.W * 4 : 0;
  if (repack_forward_ok(r)) return repack_forward_workspace(r);
  if (fast_bf16_mix_ok(r)) return r.zsave ? 0 : (size_t)r.B * r.C * r.H * r.W * 2;
  Geo g;
  if (!plan_fwd(g, r)) return 0;
  // window mode with a mix: the fp32 pre-mix map goes to z_save when that is fp32, else here
  if (r.mixw && !g.image_mode && (!r.zsave || r.out_bf16))
    return (size_t)r.B * r.C * r.H * r.W * sizeof(float);
  return 0;
}

hipError_t launch_forward(const FwdRequest& r, hipStream_t st) {
  if (hier_general(r)) return launch_forward_hier_general(r, st);  // s | w, w != 2s
  if (r.flip) {  // Z = M^T X on the general kernel (fp32 cached matrix, no mix)
    FwdArgs a{};
    if (!r.M || r.T || r.in_bf16 || r.out_bf16 || r.mixw || r.Tsub || !plan_fwd(a.g, r))
      return hipErrorInvalidValue;
    a.x = r.x;
    a.mat = r.M;
    a.zsave = r.zsave;
    a.y = r.y;
    return launch_fwd_tiles<float, 1, false, true>(a, st);
  }
  if (fast_forward_ok(r)) return launch_forward_fast(r, st);  // folds a sub-table when w = 2s
  if (!r.Tsub && fast_bf16_forward_ok(r)) return launch_forward_fast_bf16(r, st);
  // grid offset 0 or 7 on 28 x 28 and 56 x 56 maps: the rolled map
  if (fast_roll_forward_ok(r)) return launch_forward_fast_roll(r, st);
  if (fast_tab_forward_ok(r)) {  // fp32 w = 14 from the table, any map and grid offset
    if (!r.mixw) return launch_forward_fast_tab(r, (float*)r.y, (float*)r.zsave, st);
    float* z = (float*)(r.zsave ? r.zsave : r.ws);
    hipError_t e = launch_forward_fast_tab(r, z, nullptr, st);
    if (e != hipSuccess) return e;
    return launch_mix_fwd_f32_route(z, r.mixw, (float*)r.y, r.B, r.C, r.H, r.W, st);
  }
  if (repack_forward_ok(r)) return launch_forward_repacked(r, st);  // offset grid, w = 14
  if (fast_cm_forward_ok(r)) {  // cached matrix, fp32, w = 14: the contraction, then the mix pass
    if (!r.mixw) return launch_forward_fast_cm(r, (float*)r.y, (float*)r.zsave, st);
    float* z = (float*)(r.zsave ? r.zsave : r.ws);
    hipError_t e = launch_forward_fast_cm(r, z, nullptr, st);
    if (e != hipSuccess) return e;
    return launch_mix_fwd_f32_route(z, r.mixw, (float*)r.y, r.B, r.C, r.H, r.W, st);
  }
  // fp32, w = 7 or 28, 56x56: the contraction, then the mix pass
  const bool f7 = fast_f32_w7_forward_ok(r), f28 = fast_f32_w28_forward_ok(r);
  if (f7 || f28) {
    auto contract = [&](float* out, float* out2) {
      return f7 ? launch_forward_fast_f32_w7(r, out, out2, st)
                : launch_forward_fast_f32_w28(r, out, out2, st);
    };
    if (!r.mixw) return contract((float*)r.y, (float*)r.zsave);
    float* z = (float*)(r.zsave ? r.zsave : r.ws);
    hipError_t e = contract(z, nullptr);
    if (e != hipSuccess) return e;
    return launch_mix_fwd_f32_route(z, r.mixw, (float*)r.y, r.B, r.C, r.H, r.W, st);
  }
  if (fast_bf16_fused_mix_ok(r)) return launch_forward_fast_bf16_mix(r, st);  // w = 14
  if (fast_bf16_mix_ok(r)) {
    FwdRequest q = r;
    uint16_t* zb = (uint16_t*)(r.zsave ? r.zsave : r.ws);
    q.mixw = nullptr;
    q.zsave = nullptr;
    q.y = zb;
    hipError_t e = launch_forward_fast_bf16(q, st);
    if (e != hipSuccess) return e;
    return launch_mix_fwd_planes_bf16(zb, r.mixw, (uint16_t*)r.y, r.B, r.C, r.H, r.W, st);
  }
  FwdArgs a{};
  if (!plan_fwd(a.g, r)) return hipErrorInvalidValue;
  a.x = r.x;
  a.tab = r.T;
  a.tsub = r.Tsub;
  a.mat = r.M;
  a.mixw = r.mixw;
  a.out_bf16 = r.out_bf16;
  const bool mix = r.mixw != nullptr;
  float* zbuf = nullptr;
  if (a.g.image_mode) {
    a.zsave = r.zsave;
    a.y = r.y;
    a.mix_here = mix ? 1 : 0;
  } else if (mix) {
    // pre-mix output goes to an fp32 z_save or to the workspace (a bf16 z_save is written from it
    // by the mix pass)
    zbuf = (r.zsave && !r.out_bf16) ? (float*)r.zsave : (float*)r.ws;
    a.zsave = nullptr;
    a.y = zbuf;
    a.out_bf16 = 0;
    a.mix_here = 0;
  } else {
    a.zsave = r.zsave;
    a.y = r.y;
    a.mix_here = 0;
  }
  const bool cached = r.M != nullptr;
  hipError_t e;
  if (r.Tsub) e = launch_fwd_tiles<float, 0, true>(a, st);  // fp32 table path only (planned so)
  else if (r.in_bf16) e = cached ? launch_fwd_tiles<uint16_t, 1>(a, st) : launch_fwd_tiles<uint16_t, 0>(a, st);
  else e = cached ? launch_fwd_tiles<float, 1>(a, st) : launch_fwd_tiles<float, 0>(a, st);
  if (e != hipSuccess) return e;
  if (!a.g.image_mode && mix) {
    if (!r.out_bf16 && r.layout == 0)
      return launch_mix_fwd_f32_route(zbuf, r.mixw, (float*)r.y, r.B, r.C, r.H, r.W, st);
    e = launch_mix_fwd(zbuf, r.mixw, r.y, r.out_bf16, r.B, r.C, r.H, r.W, r.layout, st,
                       (r.zsave && r.out_bf16) ? (uint16_t*)r.zsave : nullptr);
  }
  return e;
}

}  // namespace wbmm
