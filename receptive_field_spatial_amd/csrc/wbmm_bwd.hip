// WBMM backward on gfx950 (fp32). The pages train with the operator but leave its backward
// implicit; by the chain rule (forward z = M_c . X_c per window, y = mix3x3(z)):
//   dz  = mix adjoint of dy;  dWmix[c,u,t] = sum dy[h,v] z[h+u-1, v+t-1];
//   dX  = M_c^T . G_c  (G = partition(dz));  dT_c[k] = sum_{idx[i][j] = k} (G_c . X_c^T)[i][j].
// One kernel does all of it in image mode: dz is formed in LDS from dy, dX reuses the forward
// contraction with the transposed table lookup, and dT is a row-pair MFMA contraction
//   acc_dy[x1][x2] = sum_{windows n} sum_{y1 - y2 = dy} G_n[y1][x1] * X_n[y2][x2]
// whose diagonals x1 - x2 = dx give dT[dy][dx]. fp32 MFMA chains over 4 windows are promoted to
// fp64; per-workgroup fp64 partials are summed in a fixed order by a small second kernel (no
// floating-point atomics, no cross-workgroup fences), so dT and dWmix are bitwise reproducible.
#include "wbmm_core.hpp"
#include "wbmm_launch.hpp"

namespace wbmm {

// Maps (x, dy or dz, z, dx) and the table are fp32, or bf16 (TM = uint16_t: mixed-precision
// training on the general shapes); the tiles and MFMAs are fp32 either way (bf16 values widen
// exactly, their products are exact in fp32), dx is rounded to the map type.
struct BwdArgs {
  Geo g;
  const void* x;
  const void* tab;
  const float* mat;
  const float* mixw;
  const void* zsaved;
  const void* gsrc;     // dy (mix applied here, or no mix) or dz (mix applied by a prior pass)
  void* dx;
  float* dT;
  float* dmixw;
  double* partT;        // [C][col_groups][L]
  double* partW;        // [C][col_groups][9]
  int mix_here, want_dx, want_dT, want_dW;
  const float* tsub;    // sub-window tables folded on chip (HIER), or null
  double* partTs;       // HIER: [C][col_groups][(2s-1)^2]
  int want_dTs;
};

// Slot j of wave q covers row offset index t = 4j + (q or 3-q alternating), ordered
// 0, +1, -1, +2, -2, ...: the four waves get near-equal MFMA counts (w - |dy| per offset).
__device__ __forceinline__ int slot_dy(int j, int wave, int nd, bool& valid) {
  const int t = 4 * j + ((j & 1) ? 3 - wave : wave);
  valid = t < nd;
  return t == 0 ? 0 : ((t & 1) ? (t + 1) / 2 : -(t / 2));
}

// HIER (the on-chip fold, w = 2s): dX uses the folded matrix, and the table gradient also yields
// the sub-table's: dT_sub[dy][dx] sums (G . X^T)[i][j] over pairs inside one s x s sub-window,
// i.e. row pairs in one band of s rows (y1 / s == y2 / s) and, within them, column pairs in one
// band of s columns. Row offsets |dy| < s keep those row pairs in a second fp32 chain; dT takes
// both chains, dT_sub the second one's band-restricted diagonals.
template <int RPW, int ASRC, bool HIER = false, typename TM = float>
__global__ void __launch_bounds__(kThreads) k_wbmm_bwd(BwdArgs a) {
  constexpr int kBf16 = sizeof(TM) == 2;
  const TM* gsrc = (const TM*)a.gsrc;
  const TM* zsaved = (const TM*)a.zsaved;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ double s_wred[4][9];
  const Geo& g = a.g;
  const int c = blockIdx.y;
  const int colgrp = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int xtile_bytes = g.NT * g.XR * 4;
  float* Gt = (float*)(smem + g.lds_big);
  unsigned char* RA = smem + g.lds_big + xtile_bytes;
  float* Ts = (float*)(smem + g.lds_tab);
  int2* Offs = (int2*)(smem + g.lds_off);
  const int plane = g.PH * g.PW;

  load_table_f32<TM>(g, ASRC == 0 ? (const TM*)a.tab : nullptr, c, Ts, Offs, a.tsub);

  double wacc[9];
#pragma unroll
  for (int q = 0; q < 9; ++q) wacc[q] = 0.0;

  // ---------------------------------------------------------------- G = partition(dz)
  if (a.mix_here) {
    float* Hs = (float*)RA;  // dy planes with a one-pixel zero halo
    zero_lds(Hs, g.ipw * plane);
    zero_lds(Gt, g.NT * g.XR);
    __syncthreads();
    const int total = g.ipw * g.H * g.W;
    for (int e = threadIdx.x; e < total; e += kThreads) {
      uint32_t img, rem, h, v;
      fdivmod((uint32_t)e, g.fd_HW, img, rem);
      fdivmod(rem, g.fd_W, h, v);
      const int b = colgrp * g.ipw + (int)img;
      if (b >= g.B) continue;
      Hs[(int)img * plane + (h + 1) * g.PW + v + 1] =
          load_f32<TM>(gsrc, map_off(g.layout, b, c, (int)h, (int)v, g.C, g.H, g.W));
    }
    __syncthreads();
    float w9[9];
#pragma unroll
    for (int q = 0; q < 9; ++q) w9[q] = a.mixw[c * 9 + q];
    for (int e = threadIdx.x; e < total; e += kThreads) {
      uint32_t img, rem, p, q;
      fdivmod((uint32_t)e, g.fd_HW, img, rem);
      fdivmod(rem, g.fd_W, p, q);
      const int b = colgrp * g.ipw + (int)img;
      if (b >= g.B) continue;
      const float* P = Hs + (int)img * plane;
      // dz[p][q] = sum_{u,t} W[u][t] dy[p-u+1][q-t+1]; P holds dy shifted by the halo (+1).
      float dz = 0.f;
#pragma unroll
      for (int u = 0; u < 3; ++u)
#pragma unroll
        for (int t = 0; t < 3; ++t) dz = fmaf(w9[u * 3 + t], P[(p - u + 2) * g.PW + (q - t + 2)], dz);
      uint32_t wy, y, wx, xx;
      fdivmod(p + g.oy, g.fd_w, wy, y);
      fdivmod(q + g.ox, g.fd_w, wx, xx);
      const int n = (int)img * g.nWin + (int)wy * g.nW + (int)wx;
      Gt[xs_slot_f32(g, n, (int)y, (int)xx)] = dz;
      if (a.want_dW) {
        // dWmix[u][t] = sum_{p,q} z[p][q] * dy[p-u+1][q-t+1]
        const double zv = load_f32<TM>(zsaved, map_off(g.layout, b, c, (int)p, (int)q, g.C, g.H, g.W));
#pragma unroll
        for (int u = 0; u < 3; ++u)
#pragma unroll
          for (int t = 0; t < 3; ++t)
            wacc[u * 3 + t] += zv * (double)P[(p - u + 2) * g.PW + (q - t + 2)];
      }
    }
    __syncthreads();
  } else {
    load_xtile<TM, float>(g, gsrc, c, colgrp, Gt);
  }

  // ---------------------------------------------------------------- dX = M^T . G
  if (a.want_dx) {
    v4f acc[RPW];
    contract_f32<RPW, 1, ASRC, true, HIER>(g, c, a.mat, Gt, (float*)RA, Ts, Offs, 0, wave, acc);
    if (g.image_mode) {
      __syncthreads();
      float* St = (float*)RA;
      zero_lds(St, g.ipw * plane);
      __syncthreads();
      stage_acc<RPW>(g, colgrp, 0, wave, acc, St);
      __syncthreads();
      const int total = g.ipw * g.H * g.W;
      for (int e = threadIdx.x; e < total; e += kThreads) {
        uint32_t img, rem, h, v;
        fdivmod((uint32_t)e, g.fd_HW, img, rem);
        fdivmod(rem, g.fd_W, h, v);
        const int b = colgrp * g.ipw + (int)img;
        if (b >= g.B) continue;
        store_out(a.dx, map_off(g.layout, b, c, (int)h, (int)v, g.C, g.H, g.W),
                  St[(int)img * plane + (h + 1) * g.PW + v + 1], kBf16);
      }
    } else {
      store_acc_direct<RPW>(g, colgrp, 0, wave, acc, c, a.dx, nullptr, kBf16);
    }
  }
  __syncthreads();

  // ---------------------------------------------------------------- dT partial (row pairs)
  if (a.want_dT) {
    float* Xt = (float*)RA;
    load_xtile<TM, float>(g, (const TM*)a.x, c, colgrp, Xt);
    int nvalid;
    if (g.image_mode) {
      int imgs = g.B - colgrp * g.ipw;
      if (imgs > g.ipw) imgs = g.ipw;
      nvalid = imgs * g.nWin;
    } else {
      nvalid = g.N - colgrp * g.NT;
      if (nvalid > g.NT) nvalid = g.NT;
    }
    const int nd = 2 * g.w - 1;
    bool val[8];
    int dyv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) dyv[j] = slot_dy(j, wave, nd, val[j]);
    double acc64[8][4];
    double accs[HIER ? 8 : 1][4];  // HIER: the same-band part of slots with |dy| < s
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc64[j][r] = 0.0;
#pragma unroll
    for (int j = 0; j < (HIER ? 8 : 1); ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) accs[j][r] = 0.0;
    const int x1 = lane & 15, kn = lane >> 4;
    for (int n0 = 0; n0 < nvalid; n0 += 4) {
      const float* gcol = Gt + (n0 + kn) * g.XR + x1;
      const float* xcol = Xt + (n0 + kn) * g.XR + x1;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (!val[j]) continue;
        const int dy = dyv[j];
        const int y1s = dy > 0 ? dy : 0, y2s = dy > 0 ? 0 : -dy;
        const int cnt = g.w - (dy > 0 ? dy : -dy);
        const float* ga = gcol + y1s * g.RP;
        const float* xb = xcol + y2s * g.RP;
        if constexpr (HIER) {
          if (dy > -g.s && dy < g.s) {  // uniform
            v4f a0 = {0.f, 0.f, 0.f, 0.f}, b0 = {0.f, 0.f, 0.f, 0.f};
            for (int m = 0; m < cnt; ++m) {
              if ((y1s + m) / g.s == (y2s + m) / g.s) b0 = mfma_f32(ga[m * g.RP], xb[m * g.RP], b0);
              else a0 = mfma_f32(ga[m * g.RP], xb[m * g.RP], a0);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              acc64[j][r] += (double)a0[r] + (double)b0[r];
              accs[j][r] += (double)b0[r];
            }
            continue;
          }
        }
        v4f a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
        int m = 0;
        for (; m + 1 < cnt; m += 2) {
          a0 = mfma_f32(ga[m * g.RP], xb[m * g.RP], a0);
          a1 = mfma_f32(ga[(m + 1) * g.RP], xb[(m + 1) * g.RP], a1);
        }
        if (m < cnt) a0 = mfma_f32(ga[m * g.RP], xb[m * g.RP], a0);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc64[j][r] += (double)a0[r] + (double)a1[r];
      }
    }
    __syncthreads();  // all waves done reading the G and X tiles
    double* scr = (double*)(smem + g.lds_big) + wave * 256;
    double* pT = a.partT + ((size_t)c * g.col_groups + colgrp) * g.L;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (!val[j]) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) scr[(4 * (lane >> 4) + r) * 16 + (lane & 15)] = acc64[j][r];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (lane < nd) {
        const int dx = lane - (g.w - 1);
        double s = 0.0;
        for (int xa = 0; xa < g.w; ++xa) {
          const int xb2 = xa - dx;
          if (xb2 >= 0 && xb2 < g.w) s += scr[xa * 16 + xb2];
        }
        pT[(dyv[j] + g.w - 1) * nd + lane] = s;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    if constexpr (HIER) {
      // dT_sub partial: diagonals of the same-band tiles over column pairs in one band
      const int ns = 2 * g.s - 1;
      double* pTs = a.partTs + ((size_t)c * g.col_groups + colgrp) * ns * ns;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (!val[j] || dyv[j] <= -g.s || dyv[j] >= g.s) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) scr[(4 * (lane >> 4) + r) * 16 + (lane & 15)] = accs[j][r];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (lane < ns) {
          const int dx = lane - (g.s - 1);
          double s = 0.0;
          for (int xa = 0; xa < g.w; ++xa) {
            const int xb2 = xa - dx;
            if (xb2 >= 0 && xb2 < g.w && xa / g.s == xb2 / g.s) s += scr[xa * 16 + xb2];
          }
          pTs[(dyv[j] + g.s - 1) * ns + lane] = s;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    }
  }

  // ---------------------------------------------------------------- dWmix partial
  if (a.want_dW) {
#pragma unroll
    for (int q = 0; q < 9; ++q) {
      double v = wacc[q];
      for (int off = 32; off > 0; off >>= 1) v += __shfl_down(v, off, 64);
      if (lane == 0) s_wred[wave][q] = v;
    }
    __syncthreads();
    if (threadIdx.x < 9) {
      const int q = threadIdx.x;
      a.partW[((size_t)c * g.col_groups + colgrp) * 9 + q] =
          ((s_wred[0][q] + s_wred[1][q]) + s_wred[2][q]) + s_wred[3][q];
    }
  }

}

// ---------------------------------------------------------------------------- dispatch
template <int RPW, int ASRC, bool HIER = false, typename TM = float>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t st) {
  auto fn = k_wbmm_bwd<RPW, ASRC, HIER, TM>;
  hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     a.g.lds_total);
  if (e != hipSuccess) return e;
  return launch_main(fn, dim3(a.g.col_groups, a.g.C, 1), dim3(kThreads), a.g.lds_total, st, a);
}

template <int ASRC, bool HIER = false, typename TM = float>
static hipError_t launch_bwd_tiles(const BwdArgs& a, hipStream_t st) {
  switch (a.g.RPW) {
    case 4: return launch_bwd_t<4, ASRC, HIER, TM>(a, st);
    case 7: return launch_bwd_t<7, ASRC, HIER, TM>(a, st);
    case 13: return launch_bwd_t<13, ASRC, HIER, TM>(a, st);
    case 16: return launch_bwd_t<16, ASRC, HIER, TM>(a, st);
    default: return hipErrorInvalidValue;
  }
}

static bool plan_bwd(Geo& g, const BwdRequest& r) {
  if (r.w > 16) return false;
  const bool cached = r.M != nullptr;
  const bool mix = r.mixw != nullptr;
  const int s = r.Tsub ? r.s : 0;
  if (!plan_geo(g, r.B, r.C, r.H, r.W, r.w, r.layout, false, cached, mix, 1, s, r.oy, r.ox)) {
    if (!plan_geo(g, r.B, r.C, r.H, r.W, r.w, r.layout, false, cached, false, 1, s, r.oy, r.ox)) return false;
  }
  return g.WR == 1;
}

namespace {
struct BwdWs {
  size_t partT, partW, partTs, dz, mixp, total;
};
// Window mode with the mix on NCHW maps: the mix's data and weight gradients come from one pass
// over dy and z (G, and dWmix partials) for even widths, or odd ones whose planes fit in LDS.
bool mix_planes_route(const Geo& g, const BwdRequest& r) {
  return r.mixw && !g.image_mode && r.layout == 0 && mix_bwd_pass_ok(r.H, r.W);
}
BwdWs bwd_ws_layout(const Geo& g, const BwdRequest& r) {
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  BwdWs w{};
  w.partT = 0;
  w.partW = w.partT + al((size_t)g.C * g.col_groups * g.L * sizeof(double));
  w.partTs = w.partW + al((size_t)g.C * g.col_groups * 9 * sizeof(double));
  const size_t ls = g.s ? (size_t)(2 * g.s - 1) * (2 * g.s - 1) : 0;
  w.dz = w.partTs + al((size_t)g.C * g.col_groups * ls * sizeof(double));
  const bool need_dz = r.mixw && !g.image_mode;
  w.mixp = w.dz + (need_dz ? al((size_t)r.B * r.C * r.H * r.W * sizeof(float)) : 0);
  w.total = w.mixp +
            (mix_planes_route(g, r) ? al((size_t)r.C * mix_bwd_parts(r.B, r.H, r.W) * 9 * 8) : 0);
  return w;
}
}  // namespace

bool backward_plan_ok(const BwdRequest& r) {
  if (hier_general(r)) return hier_backward_plan_ok(r);
  if (wide_backward_ok(r)) return true;
  Geo g;
  return plan_bwd(g, r);
}

size_t backward_workspace(const BwdRequest& r) {
  if (hier_general(r)) return hier_backward_workspace(r);
  if (wide_backward_ok(r)) return backward_wide_workspace(r, sizeof(float));
  Geo g;
  if (!plan_bwd(g, r)) return 0;
  if (roll_backward_ok(r)) return roll_backward_workspace(r);
  if (repack_backward_ok(r)) return repack_backward_workspace(r);
  const size_t generic = bwd_ws_layout(g, r).total;
  const size_t fast = fast_backward_ok(r) ? fast_backward_workspace(r) : 0;
  return generic > fast ? generic : fast;
}

// The general kernels for any w <= 16, layout and map size. TM is the map type: float, or
// uint16_t for bf16 maps and table (the request's map pointers then point at bf16 data).
template <typename TM>
static hipError_t launch_backward_general(const BwdRequest& r, hipStream_t st) {
  constexpr bool kBf16 = sizeof(TM) == 2;
  BwdArgs a{};
  if (!plan_bwd(a.g, r)) return hipErrorInvalidValue;
  const BwdWs wl = bwd_ws_layout(a.g, r);
  unsigned char* ws = (unsigned char*)r.ws;
  a.x = r.x;
  a.tab = r.T;
  a.tsub = r.Tsub;
  a.partTs = (double*)(ws + wl.partTs);
  a.want_dTs = r.Tsub && r.dTsub;
  a.mat = r.M;
  a.mixw = r.mixw;
  a.zsaved = r.zsaved;
  a.dx = r.dx;
  a.dT = r.dT;
  a.dmixw = r.dmixw;
  a.partT = (double*)(ws + wl.partT);
  a.partW = (double*)(ws + wl.partW);
  a.want_dx = r.dx != nullptr;
  a.want_dT = r.dT != nullptr;
  const bool mix = r.mixw != nullptr;
  const TM* dy = (const TM*)r.dy;
  const TM* zs = (const TM*)r.zsaved;
  hipError_t e = hipSuccess;
  if (mix && !a.g.image_mode) {
    // dz (in the map type) from a separate pass, dWmix with it
    TM* dz = (TM*)(ws + wl.dz);
    if (mix_planes_route(a.g, r)) {
      double* partM = (double*)(ws + wl.mixp);
      if constexpr (kBf16)
        e = launch_mix_bwd_planes_bf16(dy, r.dmixw ? zs : nullptr, r.mixw, dz, partM, r.B, r.C,
                                       r.H, r.W, st);
      else
        e = launch_mix_bwd_planes_f32(dy, r.dmixw ? zs : nullptr, r.mixw, dz, partM, r.B, r.C,
                                      r.H, r.W, st);
      if (e != hipSuccess) return e;
      if (r.dmixw) {
        e = launch_bwd_reduce(nullptr, partM, mix_bwd_parts(r.B, r.H, r.W), r.C, 0, nullptr,
                              r.dmixw, st);
        if (e != hipSuccess) return e;
      }
    } else {
      e = launch_mix_bwd_data_t<TM>(dy, r.mixw, dz, r.B, r.C, r.H, r.W, r.layout, st);
      if (e != hipSuccess) return e;
      if (r.dmixw) {
        e = launch_mix_bwd_weight_t<TM>(dy, zs, r.dmixw, r.B, r.C, r.H, r.W, r.layout, st);
        if (e != hipSuccess) return e;
      }
    }
    a.gsrc = dz;
    a.mix_here = 0;
    a.want_dW = 0;
  } else {
    a.gsrc = dy;
    a.mix_here = mix ? 1 : 0;
    a.want_dW = (mix && r.dmixw) ? 1 : 0;
  }
  if (a.want_dTs) a.want_dT = 1;  // the sub-table gradient comes out of the table-gradient pass
  if (!a.want_dx && !a.want_dT && !a.want_dW) return hipSuccess;
  if constexpr (kBf16) {
    e = launch_bwd_tiles<0, false, uint16_t>(a, st);  // bf16 maps: table input only
  } else {
    if (r.Tsub) e = launch_bwd_tiles<0, true>(a, st);  // fp32 table path only (planned so)
    else e = r.M ? launch_bwd_tiles<1>(a, st) : launch_bwd_tiles<0>(a, st);
  }
  if (e != hipSuccess || (!a.want_dT && !a.want_dW)) return e;
  e = launch_bwd_reduce(a.partT, a.want_dW ? a.partW : nullptr, a.g.col_groups, r.C, a.g.L,
                        r.dT, a.want_dW ? r.dmixw : nullptr, st);
  if (e != hipSuccess || !a.want_dTs) return e;
  return launch_bwd_reduce(a.partTs, nullptr, a.g.col_groups, r.C,
                           (2 * a.g.s - 1) * (2 * a.g.s - 1), r.dTsub, nullptr, st);
}

hipError_t launch_backward(const BwdRequest& r, hipStream_t st) {
  if (hier_general(r)) return launch_backward_hier_general(r, st);  // s | w, w != 2s
  if (wide_backward_ok(r)) return launch_backward_wide(r, false, st);  // 16 < w <= 32
  if (fast_backward_ok(r)) return launch_backward_fast(r, st);  // folds a sub-table when w = 2s
  if (roll_backward_ok(r)) return launch_backward_rolled(r, st);  // offset 0 / 7, 28 x 28
  if (repack_backward_ok(r)) return launch_backward_repacked(r, st);  // offset grid, w = 14
  return launch_backward_general<float>(r, st);
}

// bf16 maps and table on the general kernels (the shapes the fast bf16 backward does not cover).
size_t backward_bf16_general_workspace(const BwdRequest& r) {
  if (!r.M && !r.Tsub && wide_backward_ok(r)) return backward_wide_workspace(r, 2);
  Geo g;
  if (r.M || r.Tsub || r.oy || r.ox || !plan_bwd(g, r)) return 0;
  return bwd_ws_layout(g, r).total;
}

hipError_t launch_backward_bf16_general(const BwdRequest& r, hipStream_t st) {
  if (!r.M && !r.Tsub && wide_backward_ok(r)) return launch_backward_wide(r, true, st);
  if (r.M || r.Tsub || r.oy || r.ox) return hipErrorInvalidValue;
  return launch_backward_general<uint16_t>(r, st);
}

}  // namespace wbmm
