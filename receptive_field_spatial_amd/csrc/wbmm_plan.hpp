// Launch geometry for the WBMM contraction kernels: shared by the host planner and the kernels.
//
// Work decomposition (one workgroup = 4 waves):
//   * blockIdx.y = channel c (every channel is an independent GEMM M_c . X_c);
//   * blockIdx.x = a group of columns (windows). In "image mode" a workgroup owns `ipw` whole
//     images of channel c, so the 3x3 mix can be applied to its own output in LDS; otherwise it
//     owns NT consecutive windows ("window mode").
//   * wave arrangement WR x (4/WR): WR waves split the d rows (RPW 16-row MFMA tiles each), the
//     other factor splits the columns (one 16-window MFMA column tile per wave).
//   * K is the d in-window pixels. fp32 (16x16x4 MFMA): lane group g = lane/16 walks pixels
//     k = g*KQ + s for K-step s; the X tile keeps each window's rows at pitch RP (16 or 32) so
//     that the same tile also feeds the row-pair contraction of the table gradient.
//     bf16 (16x16x32 MFMA): window rows are padded to WP (multiple of 8) pixels so that the 8
//     values a lane feeds per step are 8 consecutive pixels of one window row.
#pragma once

#include <stdint.h>
#include "wbmm_device.hpp"

namespace wbmm {

struct Geo {
  // problem
  int B, C, H, W, w, d, L, w2m1;  // L = (2w-1)^2, w2m1 = 2w-1
  int Hp, Wp, nH, nW, nWin, N;    // padded map, window grid, windows per image, per channel
  int layout;
  int s;            // hierarchical sub-window side folded on chip (w = 2s), or 0
  int oy, ox;       // window grid offset: window (wy, wx) covers map rows wy*w - oy .. and
                    // columns wx*w - ox .. (0 for the plain grid)
  // fp32 K mapping
  int KQ, RP, XR;   // K-steps, window row pitch, X-tile stride per window (floats)
  // bf16 K mapping
  int WP, KS, XSB;  // padded window row, K-steps of 32, X-tile stride per window (bf16 units)
  int CS;           // stride of one shifted table copy (bf16 units)
  // work split
  int RPW, WR, NT;  // row tiles per wave, waves along rows, windows per workgroup
  int image_mode, ipw, col_groups;
  int PH, PW;       // staging plane with a one-pixel halo: (H + 2) x (W + 2)
  int SC, MS;       // cached-M staging: K-steps per chunk, LDS row stride (elements)
  // LDS layout (bytes)
  int lds_big, lds_tab, lds_off, lds_total;
  // fast divisors
  FastDiv fd_w, fd_nW, fd_nWin, fd_W, fd_HW, fd_KQ, fd_WP, fd_d;
};

__host__ __device__ inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f{};
  f.d = d;
  f.m = d <= 1 ? 0ull : UINT64_MAX / d + 1;
  return f;
}

inline int round_up(int a, int m) { return (a + m - 1) / m * m; }

// Tile configuration for a d x d contraction: (rows per wave in 16-tiles, waves along rows).
inline void pick_tiles(int d, int& RPW, int& WR) {
  const int RT = (d + 15) / 16;
  if (RT <= 4) { RPW = 4; WR = 1; }
  else if (RT <= 7) { RPW = 7; WR = 1; }
  else if (RT <= 13) { RPW = 13; WR = 1; }
  else if (RT <= 16) { RPW = 16; WR = 1; }
  else if (RT <= 52) { RPW = 13; WR = 4; }
  else { RPW = 16; WR = 4; }
}

constexpr int kMaxLds = 160 * 1024;

// Fill the problem-dependent part of Geo. Returns false if no launch shape fits LDS.
// bf16: element type of x/T/M; cached: M read from memory (else formed from T in LDS);
// want_image: ask for image mode (needed for an in-kernel 3x3 mix);
// extra_big: bytes the caller needs in the big region beyond the X tile (backward's G tile).
// hier_s: fold an s x s sub-window table on chip (fp32 table path, w = 2s only).
// oy, ox: window grid offset, 0 <= oy, ox < w.
inline bool plan_geo(Geo& g, int B, int C, int H, int W, int w, int layout, bool bf16,
                     bool cached, bool want_image, int big_extra_tiles, int hier_s = 0,
                     int oy = 0, int ox = 0) {
  g = Geo{};
  if (hier_s && (bf16 || cached || 2 * hier_s != w)) return false;
  if (oy < 0 || ox < 0 || oy >= w || ox >= w) return false;
  g.s = hier_s;
  g.oy = oy;
  g.ox = ox;
  g.B = B; g.C = C; g.H = H; g.W = W; g.w = w; g.d = w * w;
  g.w2m1 = 2 * w - 1; g.L = g.w2m1 * g.w2m1;
  g.Hp = (H + oy + w - 1) / w * w; g.Wp = (W + ox + w - 1) / w * w;
  g.nH = g.Hp / w; g.nW = g.Wp / w; g.nWin = g.nH * g.nW; g.N = B * g.nWin;
  g.layout = layout;
  pick_tiles(g.d, g.RPW, g.WR);
  g.NT = 16 * (4 / g.WR);
  const int esz = bf16 ? 2 : 4;

  // K mapping
  g.KQ = (g.d + 3) / 4;
  g.RP = w <= 16 ? 16 : 32;
  g.XR = w * g.RP + 1;                               // slot w*RP is a zero (padded K slots)
  while (g.XR % 32 != 18) ++g.XR;                    // 16 windows land on distinct even banks
  g.WP = round_up(w, 8);
  g.KS = (w * g.WP + 31) / 32;
  g.XSB = g.KS * 32;
  while (g.XSB % 64 != 8) g.XSB += 8;                // 8 lanes x 16 B cover all 32 banks
  g.CS = round_up(g.L + 24, 8) + 8;

  // table region: fp32 -> L floats (then the folded copy with a sub-table) + offset table;
  // bf16 -> 8 shifted copies + offsets
  const int tab_bytes = bf16 ? 8 * g.CS * 2 : (hier_s ? 2 : 1) * round_up(g.L, 4) * 4;
  const int off_bytes = bf16 ? round_up(g.KS * 4, 4) * 4 : 4 * g.KQ * 8;

  // X tile (+ cached-M chunk) bytes
  const int xtile = g.NT * (bf16 ? g.XSB * 2 : g.XR * 4);
  const int rows = 16 * g.RPW * g.WR;
  if (bf16) { g.SC = 1; g.MS = 32 + 8; }
  else { g.SC = g.WR == 4 ? 2 : 8; g.MS = 4 * g.SC + 1; }
  const int mchunk = cached ? rows * g.MS * esz : 0;
  // Forward: one region holds the X tile + staged-M chunk, later the output planes.
  // Backward (big_extra_tiles = 1): the G tile, then one region that holds in turn the dy planes,
  // the staged-M chunk, the dX planes and the X tile for the table gradient.
  auto region = [&](int stage) {
    if (!big_extra_tiles) return xtile + mchunk > stage ? xtile + mchunk : stage;
    int r = xtile > mchunk ? xtile : mchunk;
    if (stage > r) r = stage;
    if (xtile + r < 8192) r = 8192 - xtile;          // per-wave fp64 reduction tiles
    return xtile + r;
  };
  int big = region(0);

  // image mode: whole images per workgroup, staged in LDS as (H+2) x (W+2) fp32 planes
  g.PH = H + 2; g.PW = W + 2;
  g.image_mode = 0; g.ipw = 0;
  const int budget = kMaxLds - tab_bytes - off_bytes - 64;
  if (want_image && g.nWin <= g.NT) {
    const int plane = g.PH * g.PW * 4;
    int ipw = g.NT / g.nWin;
    while (ipw > 0 && region(ipw * plane) > budget) --ipw;
    if (ipw > 0) {
      g.image_mode = 1;
      g.ipw = ipw;
      big = region(ipw * plane);
    }
  }
  g.col_groups = g.image_mode ? (B + g.ipw - 1) / g.ipw : (g.N + g.NT - 1) / g.NT;

  g.lds_big = 0;
  g.lds_tab = round_up(big, 16);
  g.lds_off = round_up(g.lds_tab + tab_bytes, 16);
  g.lds_total = round_up(g.lds_off + off_bytes, 16);

  g.fd_w = make_fastdiv(w);
  g.fd_nW = make_fastdiv(g.nW);
  g.fd_nWin = make_fastdiv(g.nWin);
  g.fd_W = make_fastdiv(W);
  g.fd_HW = make_fastdiv((uint32_t)(H * W));
  g.fd_KQ = make_fastdiv(g.KQ);
  g.fd_WP = make_fastdiv(g.WP);
  g.fd_d = make_fastdiv(g.d);
  return g.lds_total <= kMaxLds;
}

}  // namespace wbmm
