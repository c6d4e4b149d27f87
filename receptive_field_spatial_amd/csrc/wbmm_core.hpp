// WBMM contraction core for gfx950: window partition into LDS, M_c formed from the table in LDS
// (or staged from a cached M in memory), and the per-channel MFMA contraction Z_c = M_c . X_c
// [gecl.asia reading notes, "Core Idea": contiguous windows, table-indexed per-channel matrix,
// one batched matmul shared by all windows; "Limitation": here the matrix is formed tile by tile
// on chip instead of being materialized, which the notes list as not yet done].
#pragma once

#include "wbmm_device.hpp"
#include "wbmm_plan.hpp"

namespace wbmm {

// Workgroup-local window n_local -> (b, wy, wx); false if the column is empty.
__device__ __forceinline__ bool wg_window(const Geo& g, int colgrp, int n_local, int& b, int& wy,
                                          int& wx) {
  uint32_t q, r;
  if (g.image_mode) {
    uint32_t img, wi;
    fdivmod((uint32_t)n_local, g.fd_nWin, img, wi);
    if ((int)img >= g.ipw) return false;
    b = colgrp * g.ipw + (int)img;
    if (b >= g.B) return false;
    fdivmod(wi, g.fd_nW, q, r);
  } else {
    const int n = colgrp * g.NT + n_local;
    if (n >= g.N) return false;
    uint32_t bb, wi;
    fdivmod((uint32_t)n, g.fd_nWin, bb, wi);
    b = (int)bb;
    fdivmod(wi, g.fd_nW, q, r);
  }
  wy = (int)q;
  wx = (int)r;
  return true;
}

// LDS slot of in-window pixel (y, x) of window n in the fp32 X tile (rows at pitch RP).
__device__ __forceinline__ int xs_slot_f32(const Geo& g, int n, int y, int x) {
  return n * g.XR + y * g.RP + x;
}

// LDS slot (bf16 units) of in-window pixel (y, x) of window n in the bf16 X tile.
__device__ __forceinline__ int xs_slot_bf16(const Geo& g, int n, int y, int x) {
  return n * g.XSB + y * g.WP + x;
}

// TTile: the tile's element type (bf16 tiles feed bf16 MFMAs; a bf16 map may also be widened
// exactly into an fp32 tile).
template <typename TIn, typename TTile>
__device__ __forceinline__ void put_tile(const Geo& g, void* tile, int n, int y, int x,
                                         const TIn* __restrict__ src, size_t off) {
  if constexpr (sizeof(TTile) == 2) {
    ((uint16_t*)tile)[xs_slot_bf16(g, n, y, x)] = src[off];
  } else {
    ((float*)tile)[xs_slot_f32(g, n, y, x)] = load_f32<TIn>(src, off);
  }
}

// ---------------------------------------------------------------------------- X tile loader
// Zero the tile, then scatter channel c of the workgroup's windows into it (zero padding,
// padded K slots and empty columns stay zero). Image mode walks whole image planes so that
// global reads are contiguous rows [pith page, Fig. 2 caption: a window is one contiguous block].
// Ends with a barrier.
template <typename TIn, typename TTile = TIn>
__device__ __forceinline__ void load_xtile(const Geo& g, const TIn* __restrict__ x, int c, int colgrp,
                           void* tile) {
  constexpr bool kBf16 = sizeof(TTile) == 2;
  {
    const int words = kBf16 ? g.NT * g.XSB / 2 : g.NT * g.XR;
    uint32_t* t32 = (uint32_t*)tile;
    for (int e = threadIdx.x; e < words; e += kThreads) t32[e] = 0u;
  }
  __syncthreads();
  if (g.image_mode) {
    const int total = g.ipw * g.H * g.W;
    for (int e = threadIdx.x; e < total; e += kThreads) {
      uint32_t img, rem, h, v;
      fdivmod((uint32_t)e, g.fd_HW, img, rem);
      fdivmod(rem, g.fd_W, h, v);
      const int b = colgrp * g.ipw + (int)img;
      if (b >= g.B) continue;
      uint32_t wy, y, wx, xx;
      fdivmod(h + g.oy, g.fd_w, wy, y);
      fdivmod(v + g.ox, g.fd_w, wx, xx);
      const int n = (int)img * g.nWin + (int)wy * g.nW + (int)wx;
      put_tile<TIn, TTile>(g, tile, n, (int)y, (int)xx, x,
                           map_off(g.layout, b, c, (int)h, (int)v, g.C, g.H, g.W));
    }
  } else {
    const int total = g.NT * g.d;
    for (int e = threadIdx.x; e < total; e += kThreads) {
      uint32_t n, k, y, xx;
      fdivmod((uint32_t)e, g.fd_d, n, k);
      int b, wy, wx;
      if (!wg_window(g, colgrp, (int)n, b, wy, wx)) continue;
      fdivmod(k, g.fd_w, y, xx);
      const int h = wy * g.w + (int)y - g.oy, v = wx * g.w + (int)xx - g.ox;
      if (h < 0 || v < 0 || h >= g.H || v >= g.W) continue;
      put_tile<TIn, TTile>(g, tile, (int)n, (int)y, (int)xx, x,
                           map_off(g.layout, b, c, h, v, g.C, g.H, g.W));
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------- table setup
// fp32: Ts[q] = T_c[q] and, per (lane group gq, K-step s), the pixel k = gq*KQ + s as
//   Offs[gq*KQ + s] = { y_k*(2w-1) + x_k  (table offset; k clamped to d-1),
//                       y_k*RP + x_k      (X-tile slot; the zero slot w*RP when k >= d) }.
// With base(i) = y_i*(2w-1) + x_i + 2w(w-1), the table entry of M[i][k] is base(i) - offset and
// that of the transposed matrix (M^T, used for dX) is L-1 - base(i) + offset.
// With a sub-window side g.s (w = 2s) the hierarchical fold happens here
// [gecl.asia reading notes, "Method" point 4]: a second copy of the table at Ts + round_up(L, 4)
// holds T[q] + T_sub[q'] (one fp32 add, RNE, the same value an explicit fold stores) for the
// offsets a same-sub-window pair can have (|dy|, |dx| < s; q' is that offset in the sub-table),
// and K is walked by quadrants (lane group gq takes quadrant (gq >> 1, gq & 1)), which for
// w = 2s are exactly the sub-windows. A pair (i, k) is then inside one sub-window exactly when
// output pixel i lies in quadrant gq, so contract_f32 picks the copy per lane and tile.
// TT: the table's element type (a bf16 table is widened exactly; the fold is fp32 only).
template <typename TT = float>
__device__ __forceinline__ void load_table_f32(const Geo& g, const TT* __restrict__ T, int c, float* Ts,
                               int2* Offs, const float* __restrict__ Tsub = nullptr) {
  if (T) {
    const TT* Tc = T + (size_t)c * g.L;
    for (int q = threadIdx.x; q < g.L; q += kThreads) Ts[q] = load_f32<TT>(Tc, q);
    if (g.s) {
      const int s = g.s, s2m1 = 2 * g.s - 1;
      const float* Sc = Tsub + (size_t)c * s2m1 * s2m1;
      float* Tf = Ts + (g.L + 3) / 4 * 4;
      for (int q = threadIdx.x; q < g.L; q += kThreads) {
        const int oy = q / g.w2m1 - (g.w - 1), ox = q % g.w2m1 - (g.w - 1);
        float v = load_f32<TT>(Tc, q);
        if (oy > -s && oy < s && ox > -s && ox < s) v = v + Sc[(oy + s - 1) * s2m1 + ox + s - 1];
        Tf[q] = v;
      }
    }
  }
  for (int e = threadIdx.x; e < 4 * g.KQ; e += kThreads) {
    int k;
    if (g.s) {  // quadrant order; 4 KQ = d for even w
      const int gq = e / g.KQ, sq = e - gq * g.KQ;
      k = ((gq >> 1) * g.s + sq / g.s) * g.w + (gq & 1) * g.s + sq % g.s;
    } else {
      k = e;  // e = gq*KQ + s is exactly the pixel index
    }
    const int kc = k > g.d - 1 ? g.d - 1 : k;
    uint32_t y, xx;
    fdivmod((uint32_t)kc, g.fd_w, y, xx);
    Offs[e] = int2{(int)y * g.w2m1 + (int)xx, k < g.d ? (int)y * g.RP + (int)xx : g.w * g.RP};
  }
}

// bf16: eight copies of the reversed table R[q] = T_c[L-1-q]; copy r holds R[q] at q + r, so any
// run of 8 consecutive entries is one aligned 16-byte read from copy (-pos) & 7. Zero margins
// cover the padded pixels of each window row (whose X values are zero).
//   OffB[s*4 + gq] = y*(2w-1) + xp for padded pixel kk = s*32 + gq*8 = y*WP + xp (y clamped).
__device__ __forceinline__ void load_table_bf16(const Geo& g, const uint16_t* __restrict__ T, int c,
                                uint16_t* copies, int* OffB) {
  {
    uint32_t* c32 = (uint32_t*)copies;
    for (int e = threadIdx.x; e < 4 * g.CS; e += kThreads) c32[e] = 0u;
  }
  __syncthreads();
  const uint16_t* Tc = T + (size_t)c * g.L;
  for (int e = threadIdx.x; e < 8 * g.L; e += kThreads) {
    const int r = e / g.L, q = e - (e / g.L) * g.L;
    copies[r * g.CS + q + r] = Tc[g.L - 1 - q];
  }
  for (int e = threadIdx.x; e < 4 * g.KS; e += kThreads) {
    uint32_t y, xp;
    fdivmod((uint32_t)(e * 8), g.fd_WP, y, xp);
    if ((int)y > g.w - 1) y = g.w - 1;
    OffB[e] = (int)y * g.w2m1 + (int)xp;
  }
}

// Per-lane A-row base for MFMA row tile rt (row i = rt*16 + lane%16, clamped into the matrix).
__device__ __forceinline__ int row_base(const Geo& g, int rt, int lane) {
  int i = rt * 16 + (lane & 15);
  if (i > g.d - 1) i = g.d - 1;
  uint32_t yi, xi;
  fdivmod((uint32_t)i, g.fd_w, yi, xi);
  return (int)yi * g.w2m1 + (int)xi + 2 * g.w * (g.w - 1);
}

// ---------------------------------------------------------------------------- fp32 contraction
// acc[t] (16 x 16, rows of tile wr*RPW + t, columns ct*16..ct*16+15) = sum_k A[i][k] * X[k][n].
// ASRC 0: A from the table in LDS; ASRC 1: A staged chunk by chunk from the cached M in memory.
// FLIP: use M^T (the adjoint, for dX).
// HIER: the table path with the on-chip fold (see load_table_f32): each tile reads the folded
// copy in the lane groups whose quadrant holds the tile row's output pixel.
template <int RPW, int WR, int ASRC, bool FLIP, bool HIER = false>
__device__ __forceinline__ void contract_f32(const Geo& g, int c, const float* __restrict__ M,
                                             const float* Xs, float* Ms, const float* Ts,
                                             const int2* Offs, int wr, int ct, v4f (&acc)[RPW]) {
  const int lane = threadIdx.x & 63;
  const int gq = lane >> 4;
  const float* xcol = Xs + (ct * 16 + (lane & 15)) * g.XR;
  const int2* oc = Offs + gq * g.KQ;
#pragma unroll
  for (int t = 0; t < RPW; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};

  if constexpr (ASRC == 0) {
    int abase[RPW];
    const float* tp[RPW];
#pragma unroll
    for (int t = 0; t < RPW; ++t) {
      const int b = row_base(g, wr * RPW + t, lane);
      abase[t] = FLIP ? (g.L - 1 - b) : b;
      tp[t] = Ts;
      if constexpr (HIER) {
        int i = (wr * RPW + t) * 16 + (lane & 15);
        if (i > g.d - 1) i = g.d - 1;
        uint32_t yi, xi;
        fdivmod((uint32_t)i, g.fd_w, yi, xi);
        const int sub = ((int)yi / g.s) * 2 + (int)xi / g.s;
        if (sub == gq) tp[t] = Ts + (g.L + 3) / 4 * 4;
      }
    }
    for (int s = 0; s < g.KQ; ++s) {
      const int2 o = oc[s];
      const float bv = xcol[o.y];
#pragma unroll
      for (int t = 0; t < RPW; ++t) {
        if ((wr * RPW + t) * 16 < g.d) {
          const float av = tp[t][FLIP ? abase[t] + o.x : abase[t] - o.x];
          acc[t] = mfma_f32(av, bv, acc[t]);
        }
      }
    }
  } else {
    constexpr int SC = WR == 4 ? 2 : 8;
    constexpr int ROWS = 16 * RPW * WR;
    const size_t mbase = (size_t)c * g.d * g.d;
    for (int s0 = 0; s0 < g.KQ; s0 += SC) {
      __syncthreads();
      for (int e = threadIdx.x; e < ROWS * 4 * SC; e += kThreads) {
        int r, gg, ss;
        if constexpr (FLIP) {  // M^T[r][k] = M[k][r]: rows contiguous in memory
          r = e % ROWS;
          const int rest = e / ROWS;
          gg = rest / SC;
          ss = rest % SC;
        } else {
          r = e / (4 * SC);
          const int rest = e % (4 * SC);
          gg = rest / SC;
          ss = rest % SC;
        }
        const int s = s0 + ss, k = gg * g.KQ + s;
        float v = 0.f;
        if (r < g.d && s < g.KQ && k < g.d)
          v = FLIP ? M[mbase + (size_t)k * g.d + r] : M[mbase + (size_t)r * g.d + k];
        Ms[r * g.MS + gg * SC + ss] = v;
      }
      __syncthreads();
      const int nst = g.KQ - s0 < SC ? g.KQ - s0 : SC;
      for (int ss = 0; ss < nst; ++ss) {
        const float bv = xcol[oc[s0 + ss].y];
#pragma unroll
        for (int t = 0; t < RPW; ++t) {
          if ((wr * RPW + t) * 16 < g.d) {
            const float av = Ms[((wr * RPW + t) * 16 + (lane & 15)) * g.MS + gq * SC + ss];
            acc[t] = mfma_f32(av, bv, acc[t]);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------- bf16 contraction
template <int RPW, int WR, int ASRC>
__device__ __forceinline__ void contract_bf16(const Geo& g, int c, const uint16_t* __restrict__ M,
                                              const uint16_t* Xb, uint16_t* Mb,
                                              const uint16_t* copies, const int* OffB, int wr,
                                              int ct, v4f (&acc)[RPW]) {
  const int lane = threadIdx.x & 63;
  const int gq = lane >> 4;
  const uint16_t* xcol = Xb + (ct * 16 + (lane & 15)) * g.XSB + gq * 8;
#pragma unroll
  for (int t = 0; t < RPW; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};

  if constexpr (ASRC == 0) {
    int abase[RPW];
#pragma unroll
    for (int t = 0; t < RPW; ++t) abase[t] = g.L - 1 - row_base(g, wr * RPW + t, lane);
    for (int s = 0; s < g.KS; ++s) {
      const u32x4 bv = *(const u32x4*)(xcol + s * 32);
      const int o = OffB[s * 4 + gq];
#pragma unroll
      for (int t = 0; t < RPW; ++t) {
        if ((wr * RPW + t) * 16 < g.d) {
          const int pos = abase[t] + o;
          const int r = (-pos) & 7;
          const u32x4 av = *(const u32x4*)(copies + r * g.CS + pos + r);
          acc[t] = mfma_bf16(av, bv, acc[t]);
        }
      }
    }
  } else {
    constexpr int ROWS = 16 * RPW * WR;
    const size_t mbase = (size_t)c * g.d * g.d;
    for (int s = 0; s < g.KS; ++s) {
      __syncthreads();
      for (int e = threadIdx.x; e < ROWS * 32; e += kThreads) {
        const int r = e >> 5, kk = s * 32 + (e & 31);
        uint32_t yk, xp;
        fdivmod((uint32_t)kk, g.fd_WP, yk, xp);
        uint16_t v = 0;
        if (r < g.d && (int)yk < g.w && (int)xp < g.w)
          v = M[mbase + (size_t)r * g.d + yk * g.w + xp];
        Mb[r * g.MS + (e & 31)] = v;
      }
      __syncthreads();
      const u32x4 bv = *(const u32x4*)(xcol + s * 32);
#pragma unroll
      for (int t = 0; t < RPW; ++t) {
        if ((wr * RPW + t) * 16 < g.d) {
          const u32x4 av =
              *(const u32x4*)(Mb + ((wr * RPW + t) * 16 + (lane & 15)) * g.MS + gq * 8);
          acc[t] = mfma_bf16(av, bv, acc[t]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------- epilogue helpers
__device__ __forceinline__ void store_out(void* p, size_t off, float v, int bf16) {
  if (bf16) ((uint16_t*)p)[off] = f2bf(v);
  else ((float*)p)[off] = v;
}

// Write this wave's accumulators into the image-mode staging planes St[img][(h+1)][(v+1)]
// (positions outside the H x W map are dropped; the planes must be zeroed beforehand).
template <int RPW>
__device__ __forceinline__ void stage_acc(const Geo& g, int colgrp, int wr, int ct,
                                          const v4f (&acc)[RPW], float* St) {
  const int lane = threadIdx.x & 63;
  const int n = ct * 16 + (lane & 15);
  uint32_t img, wi, wy, wx;
  fdivmod((uint32_t)n, g.fd_nWin, img, wi);
  if ((int)img >= g.ipw || colgrp * g.ipw + (int)img >= g.B) return;
  fdivmod(wi, g.fd_nW, wy, wx);
  float* P = St + (int)img * g.PH * g.PW;
#pragma unroll
  for (int t = 0; t < RPW; ++t) {
    const int rt = wr * RPW + t;
    if (rt * 16 >= g.d) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = rt * 16 + 4 * (lane >> 4) + r;
      if (i >= g.d) continue;
      uint32_t yi, xi;
      fdivmod((uint32_t)i, g.fd_w, yi, xi);
      const int h = (int)wy * g.w + (int)yi - g.oy, v = (int)wx * g.w + (int)xi - g.ox;
      if (h >= 0 && v >= 0 && h < g.H && v < g.W) P[(h + 1) * g.PW + v + 1] = acc[t][r];
    }
  }
}

// Window mode: write accumulators straight to the map (cropped) at `out` (and `out2` if set).
template <int RPW>
__device__ __forceinline__ void store_acc_direct(const Geo& g, int colgrp, int wr, int ct,
                                                 const v4f (&acc)[RPW], int c, void* out,
                                                 void* out2, int out_bf16) {
  const int lane = threadIdx.x & 63;
  int b, wy, wx;
  if (!wg_window(g, colgrp, ct * 16 + (lane & 15), b, wy, wx)) return;
#pragma unroll
  for (int t = 0; t < RPW; ++t) {
    const int rt = wr * RPW + t;
    if (rt * 16 >= g.d) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = rt * 16 + 4 * (lane >> 4) + r;
      if (i >= g.d) continue;
      uint32_t yi, xi;
      fdivmod((uint32_t)i, g.fd_w, yi, xi);
      const int h = wy * g.w + (int)yi - g.oy, v = wx * g.w + (int)xi - g.ox;
      if (h < 0 || v < 0 || h >= g.H || v >= g.W) continue;
      const size_t off = map_off(g.layout, b, c, h, v, g.C, g.H, g.W);
      store_out(out, off, acc[t][r], out_bf16);
      if (out2) store_out(out2, off, acc[t][r], out_bf16);
    }
  }
}

// Zero n floats of LDS (workgroup-wide; caller adds the barrier).
__device__ __forceinline__ void zero_lds(float* p, int n) {
  for (int e = threadIdx.x; e < n; e += kThreads) p[e] = 0.f;
}

}  // namespace wbmm
