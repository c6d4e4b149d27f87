// Device pieces shared by the fast fp32 w = 14 kernels: the plain-grid forward and backward
// (wbmm_fast.hip) and the rolled-map kernels of offset window grids (wbmm_fastroll.hip) — the
// kernel arguments and units, the compile-time shapes, the table-operand layout of the MFMA
// contractions, the row-pair table-gradient steps and their fp64 partials, and the launch
// helpers with the LDS budget.
#pragma once

#include "wbmm_core.hpp"
#include "wbmm_launch.hpp"

namespace wbmm {

struct FastArgs {
  int B, C;
  int groups;           // units per channel: ceil(B / images per unit)
  const float* x;
  const float* T;
  const float* mixw;
  const float* zsaved;  // backward only
  const float* dy;      // backward only
  float* zsave;         // forward only
  float* y;             // forward only
  float* dx;
  float* dT;
  float* dmixw;
  double* partT;        // [C * groups][L]: one fp64 table-gradient partial per unit
  double* partW;        // [C * groups][9]
  int want_dx, want_dT, want_dW;
  const float* Tsub;    // (C, 2s-1, 2s-1) sub-window tables, s = WS / 2 (hierarchical kernels)
  double* partTs;       // [C * groups][(2s-1)^2]: sub-table gradient partials (backward)
  int want_dTs;
  int roy, rox;         // rolled kernels: window-grid offset, each 0 or WS / 2
};

constexpr int kWsThreads = 12 * 64;  // 8 consumer waves + 4 producer waves

// One unit: 4 wave-units of IPW images each (images uimg0 .. uimg0 + 4*IPW - 1) of channel c.
// Global addresses are a uniform 64-bit base (the unit's first plane, kept in scalar registers)
// plus a 32-bit per-lane element offset ir * cp + pixel, ir = image within the unit; the host
// only takes this path when every such offset fits in an int.
struct Unit {
  size_t base;  // element offset of plane (uimg0, c)
  int c, cp;    // channel; elements between the planes of consecutive images (C * plane)
  int nimg;     // images of the unit inside the batch (>= 1)
};
template <class S>
__device__ __forceinline__ Unit unit_of(const FastArgs& a, int u) {
  Unit U;
  U.c = u / a.groups;
  const int uimg0 = (u % a.groups) * 4 * S::IPW;
  U.base = ((size_t)uimg0 * a.C + U.c) * S::PLANE;
  U.cp = a.C * S::PLANE;
  const int left = a.B - uimg0;
  U.nimg = left < 4 * S::IPW ? left : 4 * S::IPW;
  return U;
}

template <int WS_, int IH_, int IW_>
struct Shape {
  static constexpr int WS = WS_, IH = IH_, IW = IW_;
  static constexpr int D = WS * WS;
  static constexpr int QW = WS / 2;            // quadrant side
  static constexpr int KQ = QW * QW;           // K-steps (pixels per lane group)
  static constexpr int RT = (D + 15) / 16;     // 16-row output tiles
  static constexpr int L1 = 2 * WS - 1;
  static constexpr int L = L1 * L1;
  static constexpr int C0 = 2 * WS * (WS - 1); // table index of offset (0,0) relative shift
  static constexpr int LP = (L + 3) / 4 * 4;   // padded table size (floats)
  static constexpr int XP = (D + 15) / 32 * 32 + 16;  // X-chunk window pitch: lane groups on disjoint banks
  static constexpr int NWY = IH / WS, NWX = IW / WS, NWIN = NWY * NWX;
  static constexpr int IPW = 16 / NWIN;        // images per wave
  static constexpr int WPITCH = D;             // floats per window in LDS
  static constexpr int RSZ = 16 * WPITCH;      // floats per wave region
  static constexpr int PLANE = IH * IW;
  static constexpr int CMAX = (QW - 1) * L1 + (QW - 1);  // largest in-quadrant table offset
  static constexpr int LS1 = 2 * QW - 1;       // sub-window table side (s = QW)
  static constexpr int LS = LS1 * LS1;
  static_assert(WS % 2 == 0 && IH % WS == 0 && IW % WS == 0 && 16 % NWIN == 0, "shape");
  static constexpr int COLS = IPW * IW;                   // image columns per wave
  static constexpr int CHUNK_IMGS = IW <= 64 ? (64 / IW < IPW ? 64 / IW : IPW) : 1;
  static constexpr int CHUNK_COLS = CHUNK_IMGS * IW;      // columns per pass (image aligned)
  static_assert(IW <= 64, "image width");
  static_assert((7 * D + 64) * 2 <= RSZ, "a wave region holds 7 fp64 row-pair tiles + a dump row");
};

// The lane index, hidden from loop-invariant code motion: per-lane address arithmetic derived
// from it is redone inside each unit step instead of being held in registers across the loop.
__device__ __forceinline__ int opaque_lane(int lane) {
  asm volatile("" : "+v"(lane));
  return lane;
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// LDS offset (window-major, within a wave region) of the window column part of image column v
// of local image im: the row part for image row h is row_part(h).
template <class S>
__device__ __forceinline__ int col_part(int im, int v) {
  return (im * S::NWIN + v / S::WS) * S::WPITCH + (v % S::WS);
}
template <class S>
__device__ constexpr int row_part(int h) {
  return (h / S::WS) * S::NWX * S::WPITCH + (h % S::WS) * S::WS;
}

// The image planes (NCHW, channel c) of one wave-unit's images, loaded into registers by `issue`
// (one image column per lane and pass) and scattered window-major into an LDS region by `commit`.
// Images at or past B read as zero. Splitting the two lets other work run while loads are in
// flight.
template <class S>
struct PlaneLoad {
  static constexpr int NP = (S::COLS + 63) / 64;
  float v[NP][S::IH];
  // src: the unit's first plane; ir0: first image of the wave-unit within the unit
  __device__ __forceinline__ void issue(const float* __restrict__ src, const Unit& U, int ir0,
                                        int lane) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int col = p * 64 + lane;
      const int cc = col < S::COLS ? col : S::COLS - 1;
      const int im = cc / S::IW, vv = cc % S::IW;
      if (ir0 + im < U.nimg) {
        const int o = (ir0 + im) * U.cp + vv;
#pragma unroll
        for (int h = 0; h < S::IH; ++h) v[p][h] = src[o + h * S::IW];
      } else {
#pragma unroll
        for (int h = 0; h < S::IH; ++h) v[p][h] = 0.f;
      }
    }
  }
  __device__ __forceinline__ void commit(float* R, int lane) const {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int col = p * 64 + lane;
      if (col < S::COLS) {
        float* dst = R + col_part<S>(col / S::IW, col % S::IW);
#pragma unroll
        for (int h = 0; h < S::IH; ++h) dst[row_part<S>(h)] = v[p][h];
      }
    }
  }
};

// Offset (dy, dx) = (q / L1, q % L1) - (WS-1) of table entry q lies in the sub-table's range.
template <class S>
__host__ __device__ constexpr bool central(int q) {
  return q / S::L1 - (S::WS - 1) > -S::QW && q / S::L1 - (S::WS - 1) < S::QW &&
         q % S::L1 - (S::WS - 1) > -S::QW && q % S::L1 - (S::WS - 1) < S::QW;
}
// Sub-table index of a central table entry q.
template <class S>
__device__ __forceinline__ int sub_index(int q) {
  return (q / S::L1 - (S::WS - 1) + S::QW - 1) * S::LS1 + (q % S::L1 - (S::WS - 1) + S::QW - 1);
}
// Sub-table entry folded into table entry q: the entry at the same offset when q is central,
// else 0. The load index is clamped, not guarded.
template <class S>
__device__ __forceinline__ float sub_entry(const float* __restrict__ Tsub, int c, int q) {
  const bool in = central<S>(q);
  const float v = Tsub[(size_t)c * S::LS + (in ? sub_index<S>(q) : 0)];
  return in ? v : 0.f;
}
// Producer thread p loads table entries p + 256 j; at most one of them is central.
template <class S>
constexpr bool one_central_per_thread() {
  for (int p = 0; p < 256; ++p) {
    int n = 0;
    for (int q = p; q < S::L; q += 256) n += central<S>(q) ? 1 : 0;
    if (n > 1) return false;
  }
  return true;
}

// One table (C, L) row into registers (producer threads ptid = 0..255) and then into LDS; with
// HIER also the central entries of the folded copy at Ts + LP (the only ones ever read there:
// pairs inside one sub-window have offsets |dy|, |dx| < s).
template <class S, bool HIER>
struct TableLoad {
  static constexpr int NT = (S::L + 255) / 256;
  static_assert(!HIER || one_central_per_thread<S>(), "one folded entry per producer thread");
  float v[NT];
  float f;  // HIER: sub-table entry of this thread's central table entry (0 if it has none)
  __device__ __forceinline__ void issue(const float* __restrict__ T,
                                        const float* __restrict__ Tsub, int c, int ptid) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int q = ptid + 256 * j;
      v[j] = q < S::L ? T[(size_t)c * S::L + q] : 0.f;
    }
    if constexpr (HIER) {
      int qc = -1;
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int q = ptid + 256 * j;
        if (q < S::L && central<S>(q)) qc = q;
      }
      const float t = Tsub[(size_t)c * S::LS + (qc >= 0 ? sub_index<S>(qc) : 0)];
      f = qc >= 0 ? t : 0.f;
    }
  }
  __device__ __forceinline__ void commit(float* Ts, int ptid) const {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int q = ptid + 256 * j;
      if (q < S::L) {
        Ts[q] = v[j];
        if constexpr (HIER) {
          if (central<S>(q)) Ts[S::LP + q] = v[j] + f;
        }
      }
    }
  }
};

// Lane geometry for the MFMA column n = lane % 16 (window n of the wave) and lane group
// gq = lane / 16 (quadrant (gq >> 1, gq & 1) of the window's pixels).
template <class S>
struct LaneGeo {
  int n, gq, qy, qx;
  __device__ LaneGeo(int lane) {
    n = lane & 15;
    gq = lane >> 4;
    qy = gq >> 1;
    qx = gq & 1;
  }
  // LDS base of this lane's quadrant in window n; pixel s of the quadrant adds kpix(s).
  __device__ int qbase() const { return n * S::WPITCH + qy * S::QW * S::WS + qx * S::QW; }
  // table offset y*(2WS-1)+x of the quadrant origin
  __device__ int qoff() const { return qy * S::QW * S::L1 + qx * S::QW; }
};
template <class S>
__device__ constexpr int kpix(int s) { return (s / S::QW) * S::WS + (s % S::QW); }
template <class S>
__device__ constexpr int ktab(int s) { return (s / S::QW) * S::L1 + (s % S::QW); }

// acc[t] = sum_s A[16(T0 + t) + lane%16][k(gq, s)] * B[k(gq, s)][n] for the NT row tiles starting
// at T0, with A from the table in LDS and B from the wave-unit's region (window n = lane % 16);
// both are single LDS reads with immediate offsets.
// Non-flipped A entry: base(i) - (qoff + ktab(s)); flipped (M^T): L-1-base(i) + qoff + ktab(s).
// HIER: rows i in the lane group's own quadrant read the folded copy at Ts + LP.
template <class S, bool FLIP, int T0, int NT, bool HIER = false>
__device__ __forceinline__ void contract(const float* Ts, const float* R, int lane,
                                         v4f (&acc)[NT]) {
  const LaneGeo<S> lg(lane);
  const float* bsrc = R + lg.qbase();
  const float* abase[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int i = (T0 + t) * 16 + (lane & 15);
    if (i > S::D - 1) i = S::D - 1;
    const int base = (i / S::WS) * S::L1 + (i % S::WS) + S::C0;
    // non-flipped address = (base - qoff - CMAX) + (CMAX - ktab(s)), both parts >= 0
    int off = FLIP ? S::L - 1 - base + lg.qoff() : base - lg.qoff() - S::CMAX;
    if constexpr (HIER) {  // an integer offset, so the pointer stays a plain LDS address
      const int qi = ((i / S::WS) / S::QW) * 2 + (i % S::WS) / S::QW;
      off += qi == lg.gq ? S::LP : 0;
    }
    abase[t] = Ts + off;
    acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int s = 0; s < S::KQ; ++s) {
    const float bv = bsrc[kpix<S>(s)];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float av = FLIP ? abase[t][ktab<S>(s)] : abase[t][S::CMAX - ktab<S>(s)];
      acc[t] = mfma_f32(av, bv, acc[t]);
    }
  }
}

// Accumulators of tiles T0 .. T0+NT-1 back into the region at the pixel positions they belong to.
template <class S, int T0, int NT>
__device__ __forceinline__ void write_acc(float* R, int lane, const v4f (&acc)[NT]) {
  float* p = R + (lane & 15) * S::WPITCH + 4 * (lane >> 4);
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (S::D % 16 != 0) {
        if ((T0 + t) * 16 + 4 * (lane >> 4) + r >= S::D) continue;
      }
      p[(T0 + t) * 16 + r] = acc[t][r];
    }
}

// One image column of a wave-unit region, as seen by the 3x3 stencils: lane `lane` of pass p owns
// column col = PW*p + lane (image im, column v). Passes are image-aligned (PW = S::CHUNK_COLS):
// the neighbour columns of an image are neighbour lanes, and a sweep that overwrites its input in
// place never rewrites a column another pass still reads. The neighbour columns' LDS bases are
// clamped to the own column at the image border and the values read there are selected away.
template <class S, int PW_ = S::CHUNK_COLS>
struct Column {
  static constexpr int PW = PW_;
  static constexpr int NP = (S::COLS + PW - 1) / PW;
  int im, v;
  bool active, hasL, hasR;
  int pc, pl, pr;  // LDS offsets (floats) of row 0 of the column and its neighbours
  __device__ __forceinline__ Column(int p, int lane) {
    const int col = p * PW + lane;
    active = lane < PW && col < S::COLS;
    const int cc = active ? col : 0;
    im = cc / S::IW;
    v = cc % S::IW;
    hasL = v > 0;
    hasR = v + 1 < S::IW;
    pc = col_part<S>(im, v);
    pl = col_part<S>(im, hasL ? v - 1 : v);
    pr = col_part<S>(im, hasR ? v + 1 : v);
  }
};

// Walk one column top to bottom with a window w[u][t] = value at (h+u-1, v+t-1) read from LDS
// (three reads per row; zero outside the image), calling f(h, w) for every row. Rows are read in blocks of RB, the next
// block's reads in flight while the current one is processed. f may overwrite row h of the
// column in LDS: every read of rows <= h+1 has been issued by then, and later blocks only read
// rows below. This form spends no VALU on the neighbours, for sweeps whose arithmetic is the
// limit; sweep_column_lanes below trades two of the reads for two DPP moves.
template <class S, int RB, class Col, class F>
__device__ __forceinline__ void sweep_column_lds(const float* R, const Col& col, F&& f) {
  static_assert(Col::PW == S::CHUNK_COLS, "image-aligned passes");
  static_assert(S::IH % RB == 0, "row block");
  auto row = [&](int h, float (&w)[3]) {
    if (h < 0 || h >= S::IH) {
      w[0] = w[1] = w[2] = 0.f;
      return;
    }
    const float l = R[col.pl + row_part<S>(h)], c = R[col.pc + row_part<S>(h)];
    const float r = R[col.pr + row_part<S>(h)];
    w[0] = col.hasL ? l : 0.f;
    w[1] = c;
    w[2] = col.hasR ? r : 0.f;
  };
  float w[3][3];
  row(-1, w[0]);
  row(0, w[1]);
  float nxt[RB][3];
#pragma unroll
  for (int j = 0; j < RB; ++j) row(j + 1, nxt[j]);
#pragma unroll
  for (int hb = 0; hb < S::IH; hb += RB) {
    float cur[RB][3];
#pragma unroll
    for (int j = 0; j < RB; ++j)
#pragma unroll
      for (int t = 0; t < 3; ++t) cur[j][t] = nxt[j][t];
    if (hb + RB < S::IH) {
#pragma unroll
      for (int j = 0; j < RB; ++j) row(hb + RB + j + 1, nxt[j]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < RB; ++j) {
#pragma unroll
      for (int t = 0; t < 3; ++t) w[2][t] = cur[j][t];
      f(hb + j, w);
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        w[0][t] = w[1][t];
        w[1][t] = w[2][t];
      }
    }
  }
}

// Walk one column top to bottom with a sliding 3x3 window w[u][t] = value at (h+u-1, v+t-1),
// calling f(h, w) for every row. Passes are image-aligned (PW = S::CHUNK_COLS), so the neighbour
// columns of a lane's column are the neighbour lanes' columns: each row costs one LDS read, the
// column's own value, and the neighbours come by wave-wide DPP shifts (a lane at an image border
// selects zero instead). Rows are read in blocks of RB, the next block's reads in flight while
// the current one is processed. f may overwrite row h of the column in LDS: every lane's reads of
// rows <= h+1 have been issued by then, and later blocks only read rows below.
__device__ __forceinline__ float lane_left(float x) {  // x of lane - 1 (wave_shr:1)
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x138, 0xf, 0xf, true));
}
__device__ __forceinline__ float lane_right(float x) {  // x of lane + 1 (wave_shl:1)
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x130, 0xf, 0xf, true));
}
template <class S, int RB, class Col, class F>
__device__ __forceinline__ void sweep_column_lanes(const float* R, const Col& col, F&& f) {
  static_assert(Col::PW == S::CHUNK_COLS, "image-aligned passes");
  static_assert(S::IH % RB == 0, "row block");
  auto ctr = [&](int h) { return (h < 0 || h >= S::IH) ? 0.f : R[col.pc + row_part<S>(h)]; };
  auto expand = [&](float c, float (&w)[3]) {
    const float l = lane_left(c), r = lane_right(c);
    w[0] = col.hasL ? l : 0.f;
    w[1] = c;
    w[2] = col.hasR ? r : 0.f;
  };
  float w[3][3];
  w[0][0] = w[0][1] = w[0][2] = 0.f;  // row -1
  expand(ctr(0), w[1]);
  float nxt[RB];
#pragma unroll
  for (int j = 0; j < RB; ++j) nxt[j] = ctr(j + 1);
#pragma unroll
  for (int hb = 0; hb < S::IH; hb += RB) {
    float cur[RB];
#pragma unroll
    for (int j = 0; j < RB; ++j) cur[j] = nxt[j];
    if (hb + RB < S::IH) {
#pragma unroll
      for (int j = 0; j < RB; ++j) nxt[j] = ctr(hb + RB + j + 1);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      expand(cur[j], w[2]);
      f(hb + j, w);
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        w[0][t] = w[1][t];
        w[1][t] = w[2][t];
      }
    }
  }
}

template <class S, bool HIER>
constexpr int table_pitch() { return HIER ? 2 * S::LP : S::LP; }

// ---------------------------------------------------------------------------- backward
// Table-gradient slots of wave Q: row offsets dy ordered 0, +1, -1, +2, -2, ... dealt in a snake
// so the four waves get near-equal MFMA counts (WS - |dy| per offset and window chunk).
template <int WS, int Q, int J>
struct Slot {
  static constexpr int ND = 2 * WS - 1;
  static constexpr int T = 4 * J + ((J & 1) ? 3 - Q : Q);
  static constexpr bool valid = T < ND;
  static constexpr int dy = T == 0 ? 0 : ((T & 1) ? (T + 1) / 2 : -(T / 2));
};

template <int WS, int Q>
__device__ constexpr bool slot_valid(int j) {
  return 4 * j + ((j & 1) ? 3 - Q : Q) < 2 * WS - 1;
}

// Row-pair contraction for the table gradient, one chunk of 4 windows (MFMA K = window):
//   acc_j[x1][x2] += sum_{y1 - y2 = dy_j} G_n[y1][x1] * X_n[y2][x2]
// G rows from the LDS regions (any wave's), X rows from the workgroup's LDS chunk buffer (4
// windows at pitch XP). Lanes with x1 or x2 >= WS produce rows/columns of acc never read.
// HIER: pairs with y1, y2 in one sub-window band (y1 / s == y2 / s, possible only for |dy| < s,
// i.e. slots j < 4) accumulate in b32[j] instead; at each flush they go to both acc64 and accs64.
// BAND: only the pairs of one band are taken (the others are not pairs of the window).
template <class S, int Q, bool HIER, bool BAND = false>
__device__ __forceinline__ void dt_chunk(const float* regions, const float* xbuf, int n0, int kn,
                                         int xc, v4f (&a32)[8], double (&acc64)[8][4],
                                         v4f (&b32)[4], double (&accs64)[4][4], bool flush) {
  constexpr int WS = S::WS;
  const int n = n0 + kn;
  const float* g = regions + (n >> 4) * S::RSZ + (n & 15) * S::WPITCH + xc;
  const float* xb = xbuf + kn * S::XP + xc;
  float Av[WS], Bv[WS];
#pragma unroll
  for (int y = 0; y < WS; ++y) {
    Av[y] = g[y * WS];
    Bv[y] = xb[y * WS];
  }
#pragma unroll
  for (int y1 = 0; y1 < WS; ++y1) {
#define WBMM_DT_STEP(J)                                                             \
  if constexpr (Slot<WS, Q, J>::valid) {                                            \
    const int y2 = y1 - Slot<WS, Q, J>::dy;                                         \
    const float bv = Bv[y2 < 0 ? 0 : (y2 < WS ? y2 : WS - 1)];                      \
    if (y2 >= 0 && y2 < WS && (!BAND || y1 / S::QW == y2 / S::QW)) {               \
      if (HIER && J < 4 && y1 / S::QW == y2 / S::QW)                                \
        b32[J & 3] = mfma_f32(Av[y1], bv, b32[J & 3]);                              \
      else                                                                          \
        a32[J] = mfma_f32(Av[y1], bv, a32[J]);                                      \
    }                                                                               \
  }
    WBMM_DT_STEP(0) WBMM_DT_STEP(1) WBMM_DT_STEP(2) WBMM_DT_STEP(3)
    WBMM_DT_STEP(4) WBMM_DT_STEP(5) WBMM_DT_STEP(6) WBMM_DT_STEP(7)
#undef WBMM_DT_STEP
  }
  if (flush) {  // promote the fp32 chains to fp64
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (!slot_valid<WS, Q>(j)) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc64[j][r] += (double)a32[j][r];
      a32[j] = v4f{0.f, 0.f, 0.f, 0.f};
      if constexpr (HIER) {
        if (j < 4) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const double b = (double)b32[j & 3][r];
            acc64[j][r] += b;
            accs64[j & 3][r] += b;
          }
          b32[j & 3] = v4f{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
  }
}

// Diagonal sums of the wave's row-pair tiles into the unit's fp64 table partial:
//   pT[dy_j][dx] = sum over x1 - x2 = dx of acc_j[x1][x2]   (x1, x2 < WS)
// Every valid tile element goes to LDS once (scr[j][x1][x2], at most 7 tiles per wave); lane
// (half, d) then sums diagonal d over half of its rows, and the two halves are added in a fixed
// order, so the result does not depend on scheduling.
template <class S, int Q>
__device__ __forceinline__ void dt_partial_write(double* scr, const double (&acc64)[8][4],
                                                 double* pT, int lane) {
  constexpr int WS = S::WS, DD = WS * WS, HALF = (WS + 1) / 2;
  const int x2 = lane & 15, g = lane >> 4;
  // elements outside the WS x WS tile go to a per-lane dump slot past the seven tiles, so the
  // stores (and the loads below) need no branches and can all be in flight together
  const int dump = 7 * DD + lane;
#define WBMM_DT_PUT(J)                                                        \
  if constexpr (Slot<WS, Q, J>::valid) {                                      \
    _Pragma("unroll") for (int r = 0; r < 4; ++r) {                           \
      const int x1 = 4 * g + r;                                               \
      scr[(x1 < WS && x2 < WS) ? J * DD + x1 * WS + x2 : dump] = acc64[J][r]; \
    }                                                                         \
  }
  WBMM_DT_PUT(0) WBMM_DT_PUT(1) WBMM_DT_PUT(2) WBMM_DT_PUT(3)
  WBMM_DT_PUT(4) WBMM_DT_PUT(5) WBMM_DT_PUT(6) WBMM_DT_PUT(7)
#undef WBMM_DT_PUT
  wave_sync_lds();
  const int h = lane >> 5, dd = lane & 31, dxv = dd - (WS - 1);
#define WBMM_DT_SUM(J)                                                        \
  if constexpr (Slot<WS, Q, J>::valid) {                                      \
    double s = 0.0;                                                           \
    _Pragma("unroll") for (int k = 0; k < HALF; ++k) {                        \
      const int x1 = h * HALF + k, xb = x1 - dxv;                             \
      const bool ok = dd < S::L1 && x1 < WS && xb >= 0 && xb < WS;            \
      const double v = scr[ok ? J * DD + x1 * WS + xb : J * DD];              \
      s += ok ? v : 0.0;                                                      \
    }                                                                         \
    const double o = __shfl_down(s, 32, 64);                                  \
    if (lane < S::L1) pT[(Slot<WS, Q, J>::dy + WS - 1) * S::L1 + lane] = s + o; \
  }
  WBMM_DT_SUM(0) WBMM_DT_SUM(1) WBMM_DT_SUM(2) WBMM_DT_SUM(3)
  WBMM_DT_SUM(4) WBMM_DT_SUM(5) WBMM_DT_SUM(6) WBMM_DT_SUM(7)
#undef WBMM_DT_SUM
}

// Sub-table gradient partial from the band tiles (slots j < 4 with |dy_j| < s):
//   pTs[dy_j + s-1][dx + s-1] = sum over x1 - x2 = dx, x1 / s == x2 / s of accs_j[x1][x2]
// The two lane halves (x1 < s, x1 >= s) are exactly the two column halves of a window; they
// are added in a fixed order as in dt_partial_write, whose LDS scratch this reuses.
template <class S, int Q>
__device__ __forceinline__ void dts_partial_write(double* scr, const double (&accs64)[4][4],
                                                  double* pTs, int lane) {
  constexpr int WS = S::WS, QW = S::QW, DD = WS * WS;
  static_assert((WS + 1) / 2 == QW, "lane halves are the column halves");
  const int x2 = lane & 15, g = lane >> 4;
  const int dump = 7 * DD + lane;
  wave_sync_lds();  // every read of the table-gradient tiles has been issued
#define WBMM_DTS_ON(J) \
  (Slot<WS, Q, J>::valid && Slot<WS, Q, J>::dy < QW && Slot<WS, Q, J>::dy > -QW)
#define WBMM_DTS_PUT(J)                                                       \
  if constexpr (WBMM_DTS_ON(J)) {                                             \
    _Pragma("unroll") for (int r = 0; r < 4; ++r) {                           \
      const int x1 = 4 * g + r;                                               \
      scr[(x1 < WS && x2 < WS) ? J * DD + x1 * WS + x2 : dump] = accs64[J][r]; \
    }                                                                         \
  }
  WBMM_DTS_PUT(0) WBMM_DTS_PUT(1) WBMM_DTS_PUT(2) WBMM_DTS_PUT(3)
#undef WBMM_DTS_PUT
  wave_sync_lds();
  const int h = lane >> 5, dd = lane & 31, dxv = dd - (QW - 1);
#define WBMM_DTS_SUM(J)                                                        \
  if constexpr (WBMM_DTS_ON(J)) {                                              \
    double s = 0.0;                                                            \
    _Pragma("unroll") for (int k = 0; k < QW; ++k) {                           \
      const int x1 = h * QW + k, xb = x1 - dxv;                                \
      const bool ok = dd < S::LS1 && xb >= h * QW && xb < (h + 1) * QW;        \
      const double v = scr[ok ? J * DD + x1 * WS + xb : J * DD];               \
      s += ok ? v : 0.0;                                                       \
    }                                                                          \
    const double o = __shfl_down(s, 32, 64);                                   \
    if (lane < S::LS1) pTs[(Slot<WS, Q, J>::dy + QW - 1) * S::LS1 + lane] = s + o; \
  }
  WBMM_DTS_SUM(0) WBMM_DTS_SUM(1) WBMM_DTS_SUM(2) WBMM_DTS_SUM(3)
#undef WBMM_DTS_SUM
#undef WBMM_DTS_ON
}

template <class S, bool HIER>
constexpr int bwd_tsz() {
  return table_pitch<S, HIER>() + 72 > 4 * S::XP ? table_pitch<S, HIER>() + 72 : 4 * S::XP;
}

// LDS is allocated to workgroups in 1280-byte granules on gfx950 (160 KiB per CU).
constexpr int kLdsPerCu = 160 * 1024, kLdsGranule = 1280;
constexpr bool lds_fits(int bytes, int wgs) {
  return (bytes + kLdsGranule - 1) / kLdsGranule * kLdsGranule * wgs <= kLdsPerCu;
}

template <class S, bool HIER = false>
constexpr int fwd_lds() { return (2 * table_pitch<S, HIER>() + 12 * S::RSZ) * 4; }
template <class S, bool HIER = false>
constexpr int bwd_lds() { return (bwd_tsz<S, HIER>() + 4 * S::RSZ) * 4; }

template <class S>
int groups(int B) { return (B + 4 * S::IPW - 1) / (4 * S::IPW); }

using S14 = Shape<14, 14, 14>;
using S28 = Shape<14, 28, 28>;
using S56 = Shape<14, 56, 56>;

// Backward: one workgroup of 4 waves per unit.
template <class S, class Fn>
hipError_t launch_ls(Fn fn, int lds, FastArgs a, hipStream_t st) {
  a.groups = groups<S>(a.B);
  const int units = a.C * a.groups;
  hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  return launch_main(fn, dim3(units), dim3(kThreads), lds, st, a);
}

}  // namespace wbmm
