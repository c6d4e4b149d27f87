// Fast fp32 WBMM forward and backward for compile-time shapes: window WS (even), image IH x IW
// (multiples of WS) in NCHW, with the images small enough that whole images fill one wave's 16
// MFMA columns (nWin = (IH/WS)(IW/WS) divides 16).
//
// Work is cut into units of 64 windows of one channel (4 wave-units of 16 windows = whole
// images). One persistent workgroup per CU walks its units in turn with two kinds of waves:
//   * 4 consumer waves (one per SIMD) run only the MFMA contractions of the current unit;
//   * 4 producer waves load the next unit (table, image planes -> window-major LDS, and in the
//     backward the mix adjoint) and run the epilogue (mix, stores) of the previous one,
// so global traffic and the 3x3 mix overlap the matrix-core work; one barrier per step.
//
// Contraction layout:
//   * the table T_c sits in LDS; M_c is never formed: each MFMA A operand is one table entry
//     picked by the pair's relative offset [gecl.asia reading notes, "Core Idea"; the notes'
//     "Limitation"/"Takeaway" name such a non-materializing kernel as future work];
//   * each wave-unit's 16 windows sit window-major in an LDS region (a window's WS*WS pixels
//     contiguous, row-major) — one contiguous block per window [pith page, Fig. 2 caption];
//   * K (the WS*WS pixels of a window) is walked as four (WS/2)x(WS/2) quadrants, one per MFMA
//     lane group, so for every K-step the table offset splits into a per-lane base plus a
//     compile-time constant: every A operand is one LDS read with an immediate offset;
//   * 3x3 mixes walk image columns with a sliding 3x3 register window (3 LDS reads per pixel).
//
// Hierarchical fold (WS = 2s): the s x s sub-windows of a window are exactly its four quadrants,
// so a pair (i, j) shares a sub-window iff quadrant(i) == quadrant(j) [gecl.asia reading notes,
// "Method", point 4]. Beside T_c the LDS holds a folded copy Tf_c = T_c + T_sub,c (the sub-table
// added at offsets |dy|, |dx| < s, one fp32 add), and an MFMA A operand comes from the copy iff
// the output pixel's quadrant equals the lane group's K quadrant: a per-lane, per-tile choice of
// base address, so the inner loops are unchanged. The backward's table-gradient pass keeps the
// row pairs of one sub-window band in chains of their own; their diagonals restricted to one
// column half give dT_sub.
#include "wbmm_core.hpp"
#include "wbmm_launch.hpp"

#include <atomic>

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

// ---------------------------------------------------------------------------- forward
// 12 waves: 8 consumers (2 per SIMD; consumer c contracts row tiles half c >> 2 of wave-unit
// c & 3) and 4 producers (wave-unit p). LDS: tables [2][TP] (by step parity; TP = LP, or 2 LP
// with the folded copy) and regions
// [3][4][RSZ] (unit k in k % 3). Step k:
//   consumers: contract unit k | barrier | accumulators -> region (z over X) | barrier
//   producers: issue loads of unit k+1, epilogue (mix, stores) of unit k-1 | barrier |
//              commit the loads | barrier
// The mid-step barrier keeps a half from overwriting X while the other half still reads it.
template <class S, bool HIER>
constexpr int table_pitch() { return HIER ? 2 * S::LP : S::LP; }

template <class S, int T0, int NT, bool HIER>
__device__ __forceinline__ void fwd_consumer(const FastArgs& a, const float* Tb, float* Rg, int wi,
                                             int nmine, int lane) {
  for (int k = -1; k <= nmine; ++k) {
    const bool work = k >= 0 && k < nmine;
    v4f acc[NT];
    float* R = Rg + (((k < 0 ? 0 : k) % 3) * 4 + wi) * S::RSZ;
    if (work) contract<S, false, T0, NT, HIER>(Tb + (k & 1) * table_pitch<S, HIER>(), R, lane, acc);
    __syncthreads();
    if (work) write_acc<S, T0, NT>(R, lane, acc);
    __syncthreads();
  }
}

// z and y = mix3x3(z) (or y = z) of one wave-unit, from the region to global memory.
template <class S, bool MIX, bool ZS>
__device__ __forceinline__ void fwd_epilogue(const FastArgs& a, const float* R, const Unit& U,
                                             int ir0, const float (&w9)[9], int lane) {
  float* yu = a.y + U.base;
  float* zu = ZS ? a.zsave + U.base : nullptr;
#pragma unroll
  for (int p = 0; p < Column<S>::NP; ++p) {
    const Column<S> col(p, lane);
    if (!col.active || ir0 + col.im >= U.nimg) continue;
    const int o = (ir0 + col.im) * U.cp + col.v;
    sweep_column_lanes<S, 7>(R, col, [&](int h, const float (&w)[3][3]) {
      const float z = w[1][1];
      if constexpr (ZS) zu[o + h * S::IW] = z;
      float yv = z;
      if constexpr (MIX) {
        yv = 0.f;
#pragma unroll
        for (int u = 0; u < 3; ++u)
#pragma unroll
          for (int t = 0; t < 3; ++t) yv = fmaf(w9[u * 3 + t], w[u][t], yv);
      }
      yu[o + h * S::IW] = yv;
    });
  }
}

template <class S, bool MIX, bool ZS, bool HIER>
__device__ __forceinline__ void fwd_producer(const FastArgs& a, float* Tb, float* Rg, int wi,
                                             int nmine, int lane, int ptid) {
  for (int k = -1; k <= nmine; ++k) {
    const bool next = k + 1 < nmine;
    float w9[9];
    Unit Up{};
    if (k >= 1) {
      Up = unit_of<S>(a, blockIdx.x + (k - 1) * gridDim.x);
      if constexpr (MIX) {
#pragma unroll
        for (int q = 0; q < 9; ++q) w9[q] = a.mixw[Up.c * 9 + q];
      }
    }
    PlaneLoad<S> pl;
    TableLoad<S, HIER> tl;
    if (next) {
      const Unit Un = unit_of<S>(a, blockIdx.x + (k + 1) * gridDim.x);
      tl.issue(a.T, a.Tsub, Un.c, ptid);
      pl.issue(a.x + Un.base, Un, wi * S::IPW, lane);
    }
    if (k >= 1)
      fwd_epilogue<S, MIX, ZS>(a, Rg + (((k - 1) % 3) * 4 + wi) * S::RSZ, Up, wi * S::IPW, w9,
                               lane);
    __syncthreads();
    if (next) {
      // with the fold's extra registers, the commit's address math is redone each step rather
      // than held across the loop
      const int tp = HIER ? opaque_lane(ptid) : ptid, pp = HIER ? opaque_lane(lane) : lane;
      tl.commit(Tb + ((k + 1) & 1) * table_pitch<S, HIER>(), tp);
      pl.commit(Rg + (((k + 1) % 3) * 4 + wi) * S::RSZ, pp);
    }
    __syncthreads();
  }
}

template <class S, bool HIER>
__global__ void __launch_bounds__(kWsThreads) k_fwd_ws(FastArgs a) {
  extern __shared__ __attribute__((aligned(16))) float smem_f[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* Tb = smem_f;
  float* Rg = smem_f + 2 * table_pitch<S, HIER>();
  const int NU = a.C * a.groups;
  const int nmine = (NU - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  // Role loops run separately, each with the same barriers per step (a workgroup barrier counts
  // wave arrivals, not program locations), so each keeps only its own registers live.
  constexpr int H0 = (S::RT + 1) / 2;
  if (wave < 4) {
    fwd_consumer<S, 0, H0, HIER>(a, Tb, Rg, wave, nmine, lane);
  } else if (wave < 8) {
    fwd_consumer<S, H0, S::RT - H0, HIER>(a, Tb, Rg, wave - 4, nmine, lane);
  } else {
    const int wi = wave - 8, ptid = threadIdx.x - 8 * 64;
    const bool mix = a.mixw != nullptr, zs = a.zsave != nullptr;
    if (mix && zs) fwd_producer<S, true, true, HIER>(a, Tb, Rg, wi, nmine, lane, ptid);
    else if (mix) fwd_producer<S, true, false, HIER>(a, Tb, Rg, wi, nmine, lane, ptid);
    else if (zs) fwd_producer<S, false, true, HIER>(a, Tb, Rg, wi, nmine, lane, ptid);
    else fwd_producer<S, false, false, HIER>(a, Tb, Rg, wi, nmine, lane, ptid);
  }
}

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

template <class S>
using BwdCol = Column<S, S::CHUNK_COLS>;

// G = partition(dz) of one wave-unit in place; dz = mix adjoint of dy (correlation with
// rot180(W)). dWmix[u][t] = sum z[p][q] dy[p-u+1][q-t+1]: the same 3x3 dy window, times z. Each
// lane walks an image column with a sliding 3x3 register window; passes are image-aligned, so no
// column's neighbours are rewritten by another pass before they are read.
template <class S, bool WANTW>
__device__ __forceinline__ void bwd_mix_sweep(float* R, const float (&w9r)[9],
                                              const float (&zpre)[BwdCol<S>::NP][S::IH],
                                              int ir0, int nimg, double (&wacc)[9], int lane) {
#pragma unroll
  for (int p = 0; p < BwdCol<S>::NP; ++p) {
    const BwdCol<S> col(p, lane);
    if (!col.active) continue;
    const bool real = ir0 + col.im < nimg;
    float wcol[9];
#pragma unroll
    for (int q = 0; q < 9; ++q) wcol[q] = 0.f;
    sweep_column_lds<S, 7>(R, col, [&](int h, const float (&w)[3][3]) {
      // w[u][t] = dy(h+u-1, v+t-1); dz(h,v) = sum_{u,t} W[2-u][2-t] w[u][t]
      float gsum = 0.f;
#pragma unroll
      for (int q = 0; q < 9; ++q) gsum = fmaf(w9r[q], w[q / 3][q % 3], gsum);
      R[col.pc + row_part<S>(h)] = gsum;
      if constexpr (WANTW) {
        const float z = real ? zpre[p][h] : 0.f;
        // dWmix[u][t] += z * dy(h-u+1, v-t+1) = z * w[2-u][2-t]
#pragma unroll
        for (int q = 0; q < 9; ++q) wcol[q] = fmaf(z, w[2 - q / 3][2 - q % 3], wcol[q]);
      }
    });
    if constexpr (WANTW) {
#pragma unroll
      for (int q = 0; q < 9; ++q) wacc[q] += (double)wcol[q];
    }
  }
}

// dX = M^T . G of the wave-unit, stored from the accumulators: lane (n, g) holds pixels
// p = 16t + 4g + r of window n, and pairs (r, r+1), r even, are neighbours in one window row
// (WS even), so each pair is one aligned 8-byte store.
template <class S>
__device__ __forceinline__ void dx_store(const FastArgs& a, const Unit& U, int ir0,
                                         const v4f (&acc)[S::RT], int lane) {
  static_assert(S::WS % 2 == 0 && S::WS > 12, "dX pair stores: even rows, at most one wrap");
  typedef float f2 __attribute__((ext_vector_type(2)));
  const int n = lane & 15, g4 = 4 * (lane >> 4);
  const int ir = ir0 + n / S::NWIN, wnd = n % S::NWIN;
  if (ir >= U.nimg) return;
  float* o = a.dx + U.base;
  const int lofs = ir * U.cp + (wnd / S::NWX) * S::WS * S::IW + (wnd % S::NWX) * S::WS + g4;
#pragma unroll
  for (int t = 0; t < S::RT; ++t)
#pragma unroll
    for (int r = 0; r < 4; r += 2) {
      const int c0 = 16 * t + r;  // p = c0 + g4
      if (c0 + g4 < S::D) {
        const int yy = c0 / S::WS + ((c0 % S::WS) + g4 >= S::WS ? 1 : 0);
        *(f2*)(o + lofs + c0 + yy * (S::IW - S::WS)) = f2{acc[t][r], acc[t][r + 1]};
      }
    }
}

// One workgroup (4 waves, one wave-unit each) per unit; three workgroups per CU. Phases:
//   dy -> G regions (mix adjoint in place, dWmix sums) | dX from the accumulators | table
//   gradient: X streamed in 4-window chunks through the table region (loads of the next chunk
//   in flight in registers), row-pair MFMAs per slot set, fp64 partial of the unit.
// Table region (floats): the table, with HIER its folded copy, then 36 doubles of dWmix sums;
// later the X chunks.
template <class S, bool HIER>
constexpr int bwd_tsz() {
  return table_pitch<S, HIER>() + 72 > 4 * S::XP ? table_pitch<S, HIER>() + 72 : 4 * S::XP;
}

template <class S, bool HIER>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(HIER ? 2 : 3, 8)))
k_bwd_ls(FastArgs a) {
  extern __shared__ __attribute__((aligned(16))) float smem_f[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* Ts = smem_f;
  // per-wave dWmix sums, [4][9] doubles, in the table region's tail (free until the X chunks)
  double* s_wred = (double*)(smem_f + table_pitch<S, HIER>());
  float* regions = smem_f + bwd_tsz<S, HIER>();
  float* R = regions + wave * S::RSZ;
  const int u = blockIdx.x;
  const Unit U = unit_of<S>(a, u);
  const int ir0 = wave * S::IPW;
  const bool mix = a.mixw != nullptr, wantW = mix && a.want_dW;

  // z for the dWmix sums (one register column per pass), table and dy, all in flight together
  float zpre[BwdCol<S>::NP][S::IH];
  if (wantW) {
    const float* zu = a.zsaved + U.base;
#pragma unroll
    for (int p = 0; p < BwdCol<S>::NP; ++p) {
      const BwdCol<S> col(p, lane);
      const int ir = ir0 + col.im < U.nimg ? ir0 + col.im : U.nimg - 1;
      const int o = ir * U.cp + col.v;
#pragma unroll
      for (int h = 0; h < S::IH; ++h) zpre[p][h] = zu[o + h * S::IW];
    }
  }
  {
    PlaneLoad<S> pl;
    pl.issue(a.dy + U.base, U, ir0, lane);
    for (int q = threadIdx.x; q < S::L; q += kThreads) {
      const float v = a.T[(size_t)U.c * S::L + q];
      Ts[q] = v;
      if constexpr (HIER) Ts[S::LP + q] = v + sub_entry<S>(a.Tsub, U.c, q);
    }
    pl.commit(R, lane);
  }
  wave_sync_lds();
  if (mix) {
    float w9r[9];
#pragma unroll
    for (int q = 0; q < 9; ++q) w9r[q] = a.mixw[(U.c * 9) + (8 - q)];  // rot180: W[2-u][2-t]
    double wacc[9];
#pragma unroll
    for (int q = 0; q < 9; ++q) wacc[q] = 0.0;
    if (wantW) {
      bwd_mix_sweep<S, true>(R, w9r, zpre, ir0, U.nimg, wacc, lane);
#pragma unroll
      for (int q = 0; q < 9; ++q) {
        double v = wacc[q];
        for (int off = 32; off > 0; off >>= 1) v += __shfl_down(v, off, 64);
        if (lane == 0) s_wred[wave * 9 + q] = v;
      }
    } else {
      bwd_mix_sweep<S, false>(R, w9r, zpre, ir0, U.nimg, wacc, lane);
    }
  }
  __syncthreads();  // table, every wave's G and the dWmix wave sums are in LDS
  if (wantW && threadIdx.x < 9) {
    const int q = threadIdx.x;
    a.partW[(size_t)u * 9 + q] = ((s_wred[q] + s_wred[9 + q]) + s_wred[18 + q]) + s_wred[27 + q];
  }

  // ---- dX = M^T . G, stored straight from the accumulators (G stays in LDS for dT)
  if (a.want_dx) {
    v4f acc[S::RT];
    contract<S, true, 0, S::RT, HIER>(Ts, R, lane, acc);
    dx_store<S>(a, U, ir0, acc, lane);
  }

  // ---- table gradient partial over the unit's 64 windows. X comes in chunks of 4 windows
  //      through the (now free) table region; the next chunk's global loads are in flight in
  //      registers while the current one is contracted.
  if (a.want_dT) {
    double acc64[8][4];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc64[j][r] = 0.0;
    v4f a32[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) a32[j] = v4f{0.f, 0.f, 0.f, 0.f};
    v4f b32[4];           // HIER: sub-window band chains of slots 0..3
    double accs64[4][4];  // HIER: their fp64 sums (the sub-table gradient tiles)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      b32[j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 4; ++r) accs64[j][r] = 0.0;
    }
    constexpr int CH_E = 4 * S::D;
    constexpr int EPT = (CH_E + kThreads - 1) / kThreads;
    // Window n = 4 ci + kn of the unit (kn = element / D) lies in image ir and window wnd with
    // ir * cp + window origin = chunk part (uniform) + element part: NWIN = 1: ir = 4 ci + kn;
    // NWIN = 4: ir = ci, wnd = kn; NWIN = 16: ir = ci / 4, window row ci % 4, column kn.
    static_assert(S::NWIN == 1 || S::NWIN == 4 || (S::NWIN == 16 && S::NWX == 4), "chunk map");
    int eoff[EPT], loff[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int e = threadIdx.x + j * kThreads;
      const int ee = e < CH_E ? e : 0;
      const int kn = ee / S::D, p = ee % S::D;
      const int pix = (p / S::WS) * S::IW + (p % S::WS);
      if constexpr (S::NWIN == 1) eoff[j] = kn * U.cp + pix;
      else if constexpr (S::NWIN == 4) eoff[j] = (kn / S::NWX) * S::WS * S::IW + (kn % S::NWX) * S::WS + pix;
      else eoff[j] = kn * S::WS + pix;
      loff[j] = e < CH_E ? kn * S::XP + p : -1;
    }
    const float* xu = a.x + U.base;
    // windows past the batch have G = 0: their loads read within the last image instead
    const int maxoff = (U.nimg - 1) * U.cp + S::PLANE - 1;
    // two register buffers: chunk ci + 2 is loaded while chunk ci is contracted, so a global
    // load has two chunks of matrix work to land (one was not enough once a CU runs only one
    // workgroup, at the end of the kernel); the loads past the last chunk repeat it (no
    // conditional loads)
    float stgA[EPT], stgB[EPT];
    auto load_chunk = [&](float (&stg)[EPT], int ci) {
      const int cbase = S::NWIN == 1 ? 4 * ci * U.cp
                        : S::NWIN == 4 ? ci * U.cp
                                       : (ci >> 2) * U.cp + (ci & 3) * S::WS * S::IW;
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        const int o = cbase + eoff[j];
        stg[j] = xu[o < maxoff ? o : maxoff];
      }
    };
    const int kn = lane >> 4, x1 = lane & 15;
    const int xc = x1 < S::WS ? x1 : S::WS - 1;
    float* xbuf = Ts;
    auto step = [&](float (&stg)[EPT], int ci) {
      if (ci > 0) __syncthreads();  // chunk ci-1 consumed by every wave
#pragma unroll
      for (int j = 0; j < EPT; ++j)
        if (loff[j] >= 0) xbuf[loff[j]] = stg[j];
      __syncthreads();
      load_chunk(stg, ci + 2 < 16 ? ci + 2 : 15);
      // fp32 chains over 4 chunks (16 windows, at most 224 products each) before each
      // promotion to fp64 (over 8 chunks the full training shape came within 7% of the
      // max-abs bound)
      const bool flush = (ci & 3) == 3;
      switch (wave) {
        case 0: dt_chunk<S, 0, HIER>(regions, xbuf, 4 * ci, kn, xc, a32, acc64, b32, accs64, flush); break;
        case 1: dt_chunk<S, 1, HIER>(regions, xbuf, 4 * ci, kn, xc, a32, acc64, b32, accs64, flush); break;
        case 2: dt_chunk<S, 2, HIER>(regions, xbuf, 4 * ci, kn, xc, a32, acc64, b32, accs64, flush); break;
        default: dt_chunk<S, 3, HIER>(regions, xbuf, 4 * ci, kn, xc, a32, acc64, b32, accs64, flush); break;
      }
    };
    load_chunk(stgA, 0);
    load_chunk(stgB, 1);
    __syncthreads();  // every wave is done with the table (dX) and the dWmix sums
    for (int ci = 0; ci < 16; ci += 2) {
      step(stgA, ci);
      step(stgB, ci + 1);
    }
    double* pT = a.partT + (size_t)u * S::L;
    __syncthreads();  // every wave is done reading the G regions and the last chunk
    double* scr = (double*)R;
    switch (wave) {
      case 0: dt_partial_write<S, 0>(scr, acc64, pT, lane); break;
      case 1: dt_partial_write<S, 1>(scr, acc64, pT, lane); break;
      case 2: dt_partial_write<S, 2>(scr, acc64, pT, lane); break;
      default: dt_partial_write<S, 3>(scr, acc64, pT, lane); break;
    }
    if constexpr (HIER) {
      if (a.want_dTs) {
        double* pTs = a.partTs + (size_t)u * S::LS;
        switch (wave) {
          case 0: dts_partial_write<S, 0>(scr, accs64, pTs, lane); break;
          case 1: dts_partial_write<S, 1>(scr, accs64, pTs, lane); break;
          case 2: dts_partial_write<S, 2>(scr, accs64, pTs, lane); break;
          default: dts_partial_write<S, 3>(scr, accs64, pTs, lane); break;
        }
      }
    }
  }
}

// ------------------------------------------------------------------- rolled offset grid
// The window grid offset by (oy, ox), each 0 or WS / 2, on IH x IW maps whose sides are multiples
// of WS (the interleaved layers of the WBMM reading notes, "Limitation": windows shifted between
// layers; pixels outside the map are zero). Rolling the map by (-oy, -ox) moves every window of
// the offset grid, as whole quadrants at their own window positions, into one window of the plain
// grid of the rolled map: a plain window in the last window row (oy != 0) holds the lower half of
// an offset window above its upper half, and likewise for the last column, so a plain window
// holds one, two or four pieces. The product keeps the pairs of one piece: the matrix is masked
// to pairs whose quadrants agree on every split axis, and the pixels outside the map, zero in the
// offset grid, are simply not there. The work is then that of the plain grid (4 windows of a 28 x
// 28 map against 9 in the offset grid).
//
// Unit = 16 images of one channel, one workgroup of 4 waves; wave k holds the plain window k
// (row-major 2 x 2) of every image of the unit in its region (image slot = MFMA column), so a
// wave's windows share one mask and the MFMA table operand stays one value per lane:
//   mask bit 1 (row split): wave's window row is the last and oy != 0; bit 0 likewise for columns;
//   pair (i, j) is kept iff ((quadrant(i) ^ quadrant(j)) & mask) == 0.
struct RollGeo {
  int cy, cx;  // rolled window origin plus offset: map row of window pixel row py is (py + cy) mod IH
  int gm;      // mask bits (2: rows split, 1: columns split)
};
template <class S>
__device__ __forceinline__ RollGeo roll_geo(const FastArgs& a, int k) {
  const int wy = k / S::NWX, wx = k % S::NWX;
  RollGeo r;
  r.cy = S::WS * wy + a.roy;
  r.cx = S::WS * wx + a.rox;
  r.gm = ((a.roy != 0 && wy == S::NWY - 1) ? 2 : 0) | ((a.rox != 0 && wx == S::NWX - 1) ? 1 : 0);
  return r;
}
__device__ __forceinline__ int wrap(int v, int n) { return v >= n ? v - n : v; }

typedef float f4a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef float f3a4 __attribute__((ext_vector_type(3), aligned(4)));
typedef float f2a4 __attribute__((ext_vector_type(2), aligned(4)));

// The 49 pixels of quadrant q of plain window k of image slot n (lane (n, q) = (lane % 16,
// lane / 16)), read from the map through the roll: 7 half-rows of QW pixels, each contiguous in
// the map (the roll moves whole quadrants), as a 16-byte and a 12-byte load. Images past the
// batch are zero. Pixel s of the quadrant is the lane's MFMA operand of K step s.
template <class S>
struct RollQuad {
  static_assert(S::QW == 7 && S::NWIN == 4 && S::IPW == 4, "28 x 28 maps of 14 x 14 windows");
  float v[S::KQ];
  __device__ __forceinline__ void load(const float* __restrict__ src, const Unit& U,
                                       const RollGeo& g, int lane) {
    const int n = lane & 15, q = lane >> 4, qy = q >> 1, qx = q & 1;
    if (n < U.nimg) {
      const float* p = src + n * U.cp + wrap(S::QW * qx + g.cx, S::IW);
#pragma unroll
      for (int r = 0; r < S::QW; ++r) {
        const float* pr = p + wrap(S::QW * qy + r + g.cy, S::IH) * S::IW;
        const f4a4 lo = *(const f4a4*)pr;
        const f3a4 hi = *(const f3a4*)(pr + 4);
        v[7 * r + 0] = lo[0]; v[7 * r + 1] = lo[1]; v[7 * r + 2] = lo[2]; v[7 * r + 3] = lo[3];
        v[7 * r + 4] = hi[0]; v[7 * r + 5] = hi[1]; v[7 * r + 6] = hi[2];
      }
    } else {
#pragma unroll
      for (int e = 0; e < S::KQ; ++e) v[e] = 0.f;
    }
  }
  // into a wave region, window-major (slot n, row-major pixels)
  __device__ __forceinline__ void commit(float* R, int lane) const {
    const LaneGeo<S> lg(lane);
    float* d = R + lg.qbase();
#pragma unroll
    for (int e = 0; e < S::KQ; ++e) d[kpix<S>(e)] = v[e];
  }
};

// Row tiles [T0, T0 + NT) of contract() with the window operand in registers and the pairs
// across pieces removed: a lane whose output quadrant and K quadrant differ on a masked axis
// reads its table operands at ZOFF, where CMAX + 1 zeros lie (an integer offset, so the address
// stays a plain LDS one; gm = 0 keeps every pair). The table operands are read two K steps
// ahead of their MFMAs, the scheduling fenced so that the reads go out first.
template <class S, bool FLIP>
__device__ constexpr int roll_koff(int s) { return FLIP ? ktab<S>(s) : S::CMAX - ktab<S>(s); }

template <class S, bool FLIP, int ZOFF, int T0, int NT>
__device__ __forceinline__ void contract_roll(const float* Ts, const float (&bq)[S::KQ], int lane,
                                              int gm, v4f (&acc)[NT]) {
  const LaneGeo<S> lg(lane);
  int rb[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int i = (T0 + t) * 16 + (lane & 15);
    if (i > S::D - 1) i = S::D - 1;
    const int base = (i / S::WS) * S::L1 + (i % S::WS) + S::C0;
    const int off = FLIP ? S::L - 1 - base + lg.qoff() : base - lg.qoff() - S::CMAX;
    const int qi = ((i / S::WS) / S::QW) * 2 + (i % S::WS) / S::QW;
    rb[t] = (((qi ^ lg.gq) & gm) == 0) ? off : ZOFF;
    acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  float a0[NT], a1[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    a0[t] = Ts[rb[t] + roll_koff<S, FLIP>(0)];
    a1[t] = Ts[rb[t] + roll_koff<S, FLIP>(1)];
  }
#pragma unroll
  for (int s = 0; s < S::KQ; s += 2) {
    float b0[NT], b1[NT];
    if (s + 2 < S::KQ) {
#pragma unroll
      for (int t = 0; t < NT; ++t) b0[t] = Ts[rb[t] + roll_koff<S, FLIP>(s + 2)];
    }
    if (s + 3 < S::KQ) {
#pragma unroll
      for (int t = 0; t < NT; ++t) b1[t] = Ts[rb[t] + roll_koff<S, FLIP>(s + 3)];
    }
    __builtin_amdgcn_sched_barrier(0);  // the reads go out before this pair's MFMAs
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = mfma_f32(a0[t], bq[s], acc[t]);
    if (s + 1 < S::KQ) {
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] = mfma_f32(a1[t], bq[s + 1], acc[t]);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      a0[t] = b0[t];
      a1[t] = b1[t];
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Accumulators of the wave's windows back to the map through the roll: lane (n, g) holds pixels
// p = 16t + 4g + r of image slot n; pairs (r, r + 1), r even, are one window row's neighbours and
// neighbours in the map unless the columns are split (the pair of pixels QW - 1, QW then lies at
// both ends of a map row), where they go as two stores. o2 (may be null) gets a second copy.
template <class S, int T0, int NT>
__device__ __forceinline__ void roll_store(float* o, float* o2, const Unit& U, const RollGeo& g,
                                           const v4f (&acc)[NT], int lane) {
  const int n = lane & 15, g4 = 4 * (lane >> 4);
  if (n >= U.nimg) return;
  const size_t ob = U.base + (size_t)n * U.cp;
  const bool split = (g.gm & 1) != 0;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 4; r += 2) {
      const int c0 = 16 * (T0 + t) + r;  // p = c0 + g4
      if (c0 + g4 >= S::D) continue;
      const int wr = (c0 % S::WS) + g4 >= S::WS ? 1 : 0;
      const int py = c0 / S::WS + wr, px = (c0 % S::WS) + g4 - wr * S::WS;
      const int row = wrap(py + g.cy, S::IH) * S::IW;
      const int e0 = row + wrap(px + g.cx, S::IW);
      if (!split) {
        *(f2a4*)(o + ob + e0) = f2a4{acc[t][r], acc[t][r + 1]};
        if (o2) *(f2a4*)(o2 + ob + e0) = f2a4{acc[t][r], acc[t][r + 1]};
      } else {
        const int e1 = row + wrap(px + 1 + g.cx, S::IW);
        o[ob + e0] = acc[t][r];
        o[ob + e1] = acc[t][r + 1];
        if (o2) {
          o2[ob + e0] = acc[t][r];
          o2[ob + e1] = acc[t][r + 1];
        }
      }
    }
}

// Forward on the offset grid: z = masked product of each wave's windows, written to y (and
// z_save); the 3 x 3 mix runs afterwards on the whole map.
// The unit's 16 pre-mix maps in LDS (map coordinates) -> y (3 x 3 mix, or a copy) and z_save.
// A thread walks an image column down the 28 rows with a 3 x 3 register window (3 LDS reads per
// pixel; the neighbour columns' reads are clamped to the own column at the image border and
// selected away); consecutive threads own consecutive columns, so the stores are row runs.
template <class S, bool MIX>
__device__ __forceinline__ void roll_epilogue(const FastArgs& a, const float* Z, const Unit& U) {
  float w9[9];
#pragma unroll
  for (int q = 0; q < 9; ++q) w9[q] = 0.f;
  if constexpr (MIX) {
#pragma unroll
    for (int q = 0; q < 9; ++q) w9[q] = a.mixw[(size_t)U.c * 9 + q];
  }
  for (int col = threadIdx.x; col < 16 * S::IW; col += kThreads) {
    const int n = col / S::IW, v = col % S::IW;
    if (n >= U.nimg) break;  // columns are image-major: the rest are past the batch too
    const float* zc = Z + n * S::PLANE + v;
    const int dl = v > 0 ? -1 : 0, dr = v < S::IW - 1 ? 1 : 0;
    const size_t ob = U.base + (size_t)n * U.cp + v;
    float up[3] = {0.f, 0.f, 0.f}, cur[3], dn[3];
    cur[0] = dl ? zc[dl] : 0.f;
    cur[1] = zc[0];
    cur[2] = dr ? zc[dr] : 0.f;
#pragma unroll
    for (int h = 0; h < S::IH; ++h) {
      if (h + 1 < S::IH) {
        const float* zr = zc + (h + 1) * S::IW;
        dn[0] = dl ? zr[dl] : 0.f;
        dn[1] = zr[0];
        dn[2] = dr ? zr[dr] : 0.f;
      } else {
        dn[0] = dn[1] = dn[2] = 0.f;
      }
      const size_t o = ob + (size_t)h * S::IW;
      if constexpr (MIX) {
        float y = 0.f;
#pragma unroll
        for (int t = 0; t < 3; ++t) y = fmaf(w9[t], up[t], y);
#pragma unroll
        for (int t = 0; t < 3; ++t) y = fmaf(w9[3 + t], cur[t], y);
#pragma unroll
        for (int t = 0; t < 3; ++t) y = fmaf(w9[6 + t], dn[t], y);
        a.y[o] = y;
      } else {
        a.y[o] = cur[1];
      }
      if (a.zsave) a.zsave[o] = cur[1];
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        up[t] = cur[t];
        cur[t] = dn[t];
      }
    }
  }
}

// Accumulators of row tiles [T0, T0 + NT) into the unit's map staging (map coordinates).
template <class S, int T0, int NT>
__device__ __forceinline__ void roll_stage(float* Z, const RollGeo& g, const v4f (&acc)[NT],
                                           int lane) {
  const int n = lane & 15, g4 = 4 * (lane >> 4);
  float* zb = Z + n * S::PLANE;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c0 = 16 * (T0 + t) + r;  // p = c0 + g4
      if (c0 + g4 >= S::D) continue;
      const int wr = (c0 % S::WS) + g4 >= S::WS ? 1 : 0;
      const int py = c0 / S::WS + wr, px = (c0 % S::WS) + g4 - wr * S::WS;
      zb[wrap(py + g.cy, S::IH) * S::IW + wrap(px + g.cx, S::IW)] = acc[t][r];
    }
}

// LDS: the table, then the unit's 16 pre-mix maps; during the products CMAX + 1 zeros for the
// masked operands sit at the end of the map staging, which is written only after every wave's
// product.
template <class S>
constexpr int roll_fwd_floats() { return S::LP + 16 * S::PLANE; }

template <class S, bool MIX>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 8)))
k_roll_fwd(FastArgs a) {
  extern __shared__ __attribute__((aligned(16))) float smem_f[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* Ts = smem_f;
  float* Z = smem_f + S::LP;
  constexpr int ZOFF = S::LP + 16 * S::PLANE - (S::CMAX + 4) / 4 * 4;
  static_assert(ZOFF >= S::LP, "zeros inside the staging");
  const Unit U = unit_of<S>(a, blockIdx.x);
  const RollGeo g = roll_geo<S>(a, wave);
  RollQuad<S> xq;
  xq.load(a.x + U.base, U, g, lane);
  for (int q = threadIdx.x; q < S::L; q += kThreads) Ts[q] = a.T[(size_t)U.c * S::L + q];
  for (int q = threadIdx.x; q <= S::CMAX; q += kThreads) Ts[ZOFF + q] = 0.f;
  __syncthreads();
  // thirds of the row tiles (5, 4, 4), held until every wave is past the zeros
  v4f acc0[5], acc1[4], acc2[4];
  contract_roll<S, false, ZOFF, 0, 5>(Ts, xq.v, lane, g.gm, acc0);
  contract_roll<S, false, ZOFF, 5, 4>(Ts, xq.v, lane, g.gm, acc1);
  contract_roll<S, false, ZOFF, 9, 4>(Ts, xq.v, lane, g.gm, acc2);
  __syncthreads();
  roll_stage<S, 0, 5>(Z, g, acc0, lane);
  roll_stage<S, 5, 4>(Z, g, acc1, lane);
  roll_stage<S, 9, 4>(Z, g, acc2, lane);
  __syncthreads();
  roll_epilogue<S, MIX>(a, Z, U);
}

// Promote the fp32 row-pair chains of one window class to fp64; with the columns split only the
// elements with x1, x2 in one column half are pairs of the layer.
template <class S, int Q>
__device__ __forceinline__ void roll_flush(v4f (&a32)[8], double (&acc64)[8][4], bool split,
                                           int lane) {
  const int x2 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (!slot_valid<S::WS, Q>(j)) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int x1 = 4 * g + r;
      const bool keep = !split || x1 / S::QW == x2 / S::QW;
      acc64[j][r] += keep ? (double)a32[j][r] : 0.0;
    }
    a32[j] = v4f{0.f, 0.f, 0.f, 0.f};
  }
}

template <class S, int Q>
__device__ __forceinline__ void roll_dt_chunk(const float* regions, const float* xbuf, int n0,
                                              int kn, int xc, bool band, v4f (&a32)[8],
                                              double (&acc64)[8][4]) {
  v4f b32[4];
  double accs64[4][4];
  if (band)
    dt_chunk<S, Q, false, true>(regions, xbuf, n0, kn, xc, a32, acc64, b32, accs64, false);
  else
    dt_chunk<S, Q, false, false>(regions, xbuf, n0, kn, xc, a32, acc64, b32, accs64, false);
}

// Backward on the offset grid (dy is the map gradient G of the product; the mix adjoint, if any,
// has run before): dX = masked M^T G per wave, stored through the roll; the table-gradient pass
// walks the unit in 16 chunks of 4 windows of one class (chunk ci: window ci / 4 of images
// 4 (ci % 4) .. +3), with the row pairs of one band only where the rows are split and the column
// mask applied when the class's chains are promoted.
template <class S>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 8)))
k_roll_bwd(FastArgs a) {
  extern __shared__ __attribute__((aligned(16))) float smem_f[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* Ts = smem_f;
  float* regions = smem_f + bwd_tsz<S, false>();
  float* R = regions + wave * S::RSZ;
  const int u = blockIdx.x;
  const Unit U = unit_of<S>(a, u);
  const RollGeo g = roll_geo<S>(a, wave);
  // G of the wave's windows in registers; during dX the zeros of the masked operands sit at the
  // start of the regions, which take G (for the table gradient) only after dX
  constexpr int ZOFF = bwd_tsz<S, false>();
  static_assert(S::CMAX < S::RSZ, "zeros inside the first region");
  RollQuad<S> gq;
  gq.load(a.dy + U.base, U, g, lane);
  for (int q = threadIdx.x; q < S::L; q += kThreads) Ts[q] = a.T[(size_t)U.c * S::L + q];
  for (int q = threadIdx.x; q <= S::CMAX; q += kThreads) Ts[ZOFF + q] = 0.f;
  __syncthreads();

  if (a.want_dx) {  // thirds of the row tiles, as in the forward
    {
      v4f acc[5];
      contract_roll<S, true, ZOFF, 0, 5>(Ts, gq.v, lane, g.gm, acc);
      roll_store<S, 0, 5>(a.dx, nullptr, U, g, acc, lane);
    }
    {
      v4f acc[4];
      contract_roll<S, true, ZOFF, 5, 4>(Ts, gq.v, lane, g.gm, acc);
      roll_store<S, 5, 4>(a.dx, nullptr, U, g, acc, lane);
    }
    {
      v4f acc[4];
      contract_roll<S, true, ZOFF, 9, 4>(Ts, gq.v, lane, g.gm, acc);
      roll_store<S, 9, 4>(a.dx, nullptr, U, g, acc, lane);
    }
  }
  if (!a.want_dT) return;
  __syncthreads();  // every wave is done with the zeros in the first region
  gq.commit(R, lane);

  {
    double acc64[8][4];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc64[j][r] = 0.0;
    v4f a32[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) a32[j] = v4f{0.f, 0.f, 0.f, 0.f};
    constexpr int CH_E = 4 * S::D;
    constexpr int EPT = (CH_E + kThreads - 1) / kThreads;
    // element e = tid + 256 j of a chunk: window kn = e / D (image 4 (ci % 4) + kn), pixel
    // p = e % D; recomputed at each use from an opaque thread index (not held across the loop)
    const float* xu = a.x + U.base;
    // windows past the batch have G = 0: their loads read within the last image instead
    const int maxoff = (U.nimg - 1) * U.cp + S::PLANE - 1;
    float stgA[EPT], stgB[EPT];
    auto load_chunk = [&](float (&stg)[EPT], int ci) {
      const RollGeo cg = roll_geo<S>(a, ci >> 2);
      const int cbase = 4 * (ci & 3) * U.cp;
      const int tid = opaque_lane(threadIdx.x);
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        const int e = tid + j * kThreads;
        const int ee = e < CH_E ? e : 0;
        const int kn = ee / S::D, p = ee % S::D;
        const int o = cbase + kn * U.cp + wrap(p / S::WS + cg.cy, S::IH) * S::IW +
                      wrap(p % S::WS + cg.cx, S::IW);
        stg[j] = xu[o < maxoff ? o : maxoff];
      }
    };
    const int kn = lane >> 4, x1 = lane & 15;
    const int xc = x1 < S::WS ? x1 : S::WS - 1;
    float* xbuf = Ts;
    auto step = [&](float (&stg)[EPT], int ci) {
      if (ci > 0) __syncthreads();  // chunk ci-1 consumed by every wave
      {
        const int tid = opaque_lane(threadIdx.x);
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
          const int e = tid + j * kThreads;
          if (e < CH_E) xbuf[(e / S::D) * S::XP + e % S::D] = stg[j];
        }
      }
      __syncthreads();
      load_chunk(stg, ci + 2 < 16 ? ci + 2 : 15);
      const RollGeo cg = roll_geo<S>(a, ci >> 2);
      const bool band = (cg.gm & 2) != 0, split = (cg.gm & 1) != 0;
      const int n0 = 16 * (ci >> 2) + 4 * (ci & 3);
      const bool flush = (ci & 3) == 3;
      switch (wave) {
        case 0:
          roll_dt_chunk<S, 0>(regions, xbuf, n0, kn, xc, band, a32, acc64);
          if (flush) roll_flush<S, 0>(a32, acc64, split, lane);
          break;
        case 1:
          roll_dt_chunk<S, 1>(regions, xbuf, n0, kn, xc, band, a32, acc64);
          if (flush) roll_flush<S, 1>(a32, acc64, split, lane);
          break;
        case 2:
          roll_dt_chunk<S, 2>(regions, xbuf, n0, kn, xc, band, a32, acc64);
          if (flush) roll_flush<S, 2>(a32, acc64, split, lane);
          break;
        default:
          roll_dt_chunk<S, 3>(regions, xbuf, n0, kn, xc, band, a32, acc64);
          if (flush) roll_flush<S, 3>(a32, acc64, split, lane);
          break;
      }
    };
    load_chunk(stgA, 0);
    load_chunk(stgB, 1);
    __syncthreads();  // every wave is done with the table (dX) and its G is in its region
    for (int ci = 0; ci < 16; ci += 2) {
      step(stgA, ci);
      step(stgB, ci + 1);
    }
    double* pT = a.partT + (size_t)u * S::L;
    __syncthreads();  // every wave is done reading the G regions and the last chunk
    double* scr = (double*)R;
    switch (wave) {
      case 0: dt_partial_write<S, 0>(scr, acc64, pT, lane); break;
      case 1: dt_partial_write<S, 1>(scr, acc64, pT, lane); break;
      case 2: dt_partial_write<S, 2>(scr, acc64, pT, lane); break;
      default: dt_partial_write<S, 3>(scr, acc64, pT, lane); break;
    }
  }
}

// ---------------------------------------------------------------------------- dispatch
namespace {

// Shapes with a compiled fast path: (window, image height, image width).
enum FastShape { FS_NONE, FS_14_14_14, FS_14_28_28, FS_14_56_56 };

FastShape fast_shape(int H, int W, int w, int layout) {
  if (layout != 0 || w != 14) return FS_NONE;
  if (H == 14 && W == 14) return FS_14_14_14;
  if (H == 28 && W == 28) return FS_14_28_28;
  if (H == 56 && W == 56) return FS_14_56_56;
  return FS_NONE;
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

// Compute units of the current device (cached per device); one persistent workgroup per CU.
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <class S, class Fn>
hipError_t launch_ws(Fn fn, int lds, FastArgs a, hipStream_t st) {
  a.groups = groups<S>(a.B);
  const int units = a.C * a.groups;
  const int cus = cu_count();
  const int grid = units < cus ? units : cus;
  hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  return launch_main(fn, dim3(grid), dim3(kWsThreads), lds, st, a);
}

using S14 = Shape<14, 14, 14>;
using S28 = Shape<14, 28, 28>;
using S56 = Shape<14, 56, 56>;
static_assert(lds_fits(fwd_lds<S14>(), 1) && lds_fits(fwd_lds<S28>(), 1) &&
                  lds_fits(fwd_lds<S56>(), 1),
              "one persistent forward workgroup per CU");
static_assert(lds_fits(bwd_lds<S14>(), 3) && lds_fits(bwd_lds<S28>(), 3) &&
                  lds_fits(bwd_lds<S56>(), 3),
              "three backward workgroups per CU");
// with the folded table copy: still one persistent forward workgroup, two backward per CU
static_assert(lds_fits(fwd_lds<S14, true>(), 1) && lds_fits(fwd_lds<S28, true>(), 1) &&
                  lds_fits(fwd_lds<S56, true>(), 1),
              "one persistent hierarchical forward workgroup per CU");
static_assert(lds_fits(bwd_lds<S14, true>(), 2) && lds_fits(bwd_lds<S28, true>(), 2) &&
                  lds_fits(bwd_lds<S56, true>(), 2),
              "two hierarchical backward workgroups per CU");
template <class S>
constexpr int roll_fwd_lds() { return roll_fwd_floats<S>() * 4; }
static_assert(lds_fits(roll_fwd_lds<S28>(), 3) && lds_fits(bwd_lds<S28>(), 3),
              "three rolled-grid workgroups per CU");

// Backward: one workgroup of 4 waves per unit.
template <class S, class Fn>
hipError_t launch_ls(Fn fn, int lds, FastArgs a, hipStream_t st) {
  a.groups = groups<S>(a.B);
  const int units = a.C * a.groups;
  hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  return launch_main(fn, dim3(units), dim3(kThreads), lds, st, a);
}

}  // namespace

// Per-lane offsets within a unit are ints: ir * C * plane + pixel, ir < 16 images.
bool offsets_fit(int C, int H, int W) { return (size_t)16 * C * H * W < ((size_t)1 << 31); }

// A sub-table is folded on chip when its sub-windows are the quadrants (w = 2s).
bool fast_forward_ok(const FwdRequest& r) {
  return !r.in_bf16 && !r.out_bf16 && r.T && !r.M && (!r.Tsub || 2 * r.s == r.w) &&
         r.oy == 0 && r.ox == 0 &&
         fast_shape(r.H, r.W, r.w, r.layout) != FS_NONE && offsets_fit(r.C, r.H, r.W);
}

bool fast_backward_ok(const BwdRequest& r) {
  return r.T && !r.M && (!r.Tsub || 2 * r.s == r.w) && r.oy == 0 && r.ox == 0 &&
         fast_shape(r.H, r.W, r.w, r.layout) != FS_NONE && offsets_fit(r.C, r.H, r.W);
}

hipError_t launch_forward_fast(const FwdRequest& r, hipStream_t st) {
  FastArgs a{};
  a.B = r.B;
  a.C = r.C;
  a.x = (const float*)r.x;
  a.T = (const float*)r.T;
  a.mixw = r.mixw;
  a.zsave = (float*)r.zsave;
  a.y = (float*)r.y;
  a.Tsub = r.Tsub;
  const bool h = r.Tsub != nullptr;
  switch (fast_shape(r.H, r.W, r.w, r.layout)) {
    case FS_14_14_14:
      return h ? launch_ws<S14>(k_fwd_ws<S14, true>, fwd_lds<S14, true>(), a, st)
               : launch_ws<S14>(k_fwd_ws<S14, false>, fwd_lds<S14>(), a, st);
    case FS_14_28_28:
      return h ? launch_ws<S28>(k_fwd_ws<S28, true>, fwd_lds<S28, true>(), a, st)
               : launch_ws<S28>(k_fwd_ws<S28, false>, fwd_lds<S28>(), a, st);
    case FS_14_56_56:
      return h ? launch_ws<S56>(k_fwd_ws<S56, true>, fwd_lds<S56, true>(), a, st)
               : launch_ws<S56>(k_fwd_ws<S56, false>, fwd_lds<S56>(), a, st);
    default: return hipErrorInvalidValue;
  }
}

// The offset grid on the rolled map: fp32, w = 14, NCHW 28 x 28, offsets 0 or 7 (not both 0).
static bool roll_shape_ok(int B, int C, int H, int W, int w, int layout, int oy, int ox) {
  return w == 14 && layout == 0 && H == 28 && W == 28 && (oy == 0 || oy == 7) &&
         (ox == 0 || ox == 7) && (oy != 0 || ox != 0) && B >= 1 && C >= 1 &&
         offsets_fit(C, H, W);
}

bool fast_roll_forward_ok(const FwdRequest& r) {
  return !r.in_bf16 && !r.out_bf16 && r.T && !r.M && !r.Tsub && !r.flip &&
         roll_shape_ok(r.B, r.C, r.H, r.W, r.w, r.layout, r.oy, r.ox);
}

bool fast_roll_backward_ok(const BwdRequest& r) {
  return r.T && !r.M && !r.Tsub && roll_shape_ok(r.B, r.C, r.H, r.W, r.w, r.layout, r.oy, r.ox);
}

// The layer on the offset grid: y (with the 3 x 3 mix applied on chip when there is one) and
// z_save (the pre-mix map), both optional-free: y is always written.
hipError_t launch_forward_fast_roll(const FwdRequest& r, hipStream_t st) {
  if (!fast_roll_forward_ok(r)) return hipErrorInvalidValue;
  FastArgs a{};
  a.B = r.B;
  a.C = r.C;
  a.x = (const float*)r.x;
  a.T = (const float*)r.T;
  a.mixw = r.mixw;
  a.y = (float*)r.y;
  a.zsave = (float*)r.zsave;
  a.roy = r.oy;
  a.rox = r.ox;
  return r.mixw ? launch_ls<S28>(k_roll_fwd<S28, true>, roll_fwd_lds<S28>(), a, st)
                : launch_ls<S28>(k_roll_fwd<S28, false>, roll_fwd_lds<S28>(), a, st);
}

// Table-gradient partials of the rolled backward: one fp64 row of L per unit.
size_t fast_roll_backward_workspace(const BwdRequest& r) {
  if (!fast_roll_backward_ok(r)) return 0;
  const size_t L = (size_t)(2 * r.w - 1) * (2 * r.w - 1);
  return ((size_t)r.C * groups<S28>(r.B) * L * 8 + 255) / 256 * 256;
}

// dy: the map gradient of the product (the mix adjoint, if any, already applied).
hipError_t launch_backward_fast_roll(const BwdRequest& r, hipStream_t st) {
  if (!fast_roll_backward_ok(r)) return hipErrorInvalidValue;
  FastArgs a{};
  a.B = r.B;
  a.C = r.C;
  a.x = r.x;
  a.T = r.T;
  a.dy = r.dy;
  a.dx = r.dx;
  a.dT = r.dT;
  a.partT = (double*)r.ws;
  a.want_dx = r.dx != nullptr;
  a.want_dT = r.dT != nullptr;
  a.roy = r.oy;
  a.rox = r.ox;
  if (!a.want_dx && !a.want_dT) return hipSuccess;
  hipError_t e = launch_ls<S28>(k_roll_bwd<S28>, bwd_lds<S28>(), a, st);
  if (e != hipSuccess || !a.want_dT) return e;
  const int L = (2 * r.w - 1) * (2 * r.w - 1);
  return launch_bwd_reduce(a.partT, nullptr, groups<S28>(r.B), r.C, L, r.dT, nullptr, st);
}

size_t fast_backward_workspace(const BwdRequest& r) {
  int g;
  switch (fast_shape(r.H, r.W, r.w, r.layout)) {
    case FS_14_14_14: g = groups<S14>(r.B); break;
    case FS_14_28_28: g = groups<S28>(r.B); break;
    case FS_14_56_56: g = groups<S56>(r.B); break;
    default: return 0;
  }
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  const size_t L = (size_t)(2 * r.w - 1) * (2 * r.w - 1);
  const size_t Ls = r.Tsub ? (size_t)(2 * r.s - 1) * (2 * r.s - 1) : 0;
  return al((size_t)r.C * g * L * 8) + al((size_t)r.C * g * 9 * 8) + al((size_t)r.C * g * Ls * 8);
}

hipError_t launch_backward_fast(const BwdRequest& r, hipStream_t st) {
  FastArgs a{};
  a.B = r.B;
  a.C = r.C;
  int g;
  const FastShape fs = fast_shape(r.H, r.W, r.w, r.layout);
  switch (fs) {
    case FS_14_14_14: g = groups<S14>(r.B); break;
    case FS_14_28_28: g = groups<S28>(r.B); break;
    case FS_14_56_56: g = groups<S56>(r.B); break;
    default: return hipErrorInvalidValue;
  }
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  const size_t L = (size_t)(2 * r.w - 1) * (2 * r.w - 1);
  unsigned char* ws = (unsigned char*)r.ws;
  a.partT = (double*)ws;
  a.partW = (double*)(ws + al((size_t)r.C * g * L * 8));
  a.partTs = (double*)(ws + al((size_t)r.C * g * L * 8) + al((size_t)r.C * g * 9 * 8));
  a.Tsub = r.Tsub;
  a.x = r.x;
  a.T = r.T;
  a.mixw = r.mixw;
  a.zsaved = r.zsaved;
  a.dy = r.dy;
  a.dx = r.dx;
  a.dT = r.dT;
  a.dmixw = r.dmixw;
  a.want_dx = r.dx != nullptr;
  a.want_dT = r.dT != nullptr;
  a.want_dW = (r.mixw && r.dmixw) ? 1 : 0;
  a.want_dTs = (r.Tsub && r.dTsub) ? 1 : 0;
  if (a.want_dTs) a.want_dT = 1;  // the sub-table gradient comes out of the table-gradient pass
  if (!a.want_dx && !a.want_dT && !a.want_dW) return hipSuccess;
  const bool h = r.Tsub != nullptr;
  hipError_t e;
  switch (fs) {
    case FS_14_14_14:
      e = h ? launch_ls<S14>(k_bwd_ls<S14, true>, bwd_lds<S14, true>(), a, st)
            : launch_ls<S14>(k_bwd_ls<S14, false>, bwd_lds<S14>(), a, st);
      break;
    case FS_14_28_28:
      e = h ? launch_ls<S28>(k_bwd_ls<S28, true>, bwd_lds<S28, true>(), a, st)
            : launch_ls<S28>(k_bwd_ls<S28, false>, bwd_lds<S28>(), a, st);
      break;
    default:
      e = h ? launch_ls<S56>(k_bwd_ls<S56, true>, bwd_lds<S56, true>(), a, st)
            : launch_ls<S56>(k_bwd_ls<S56, false>, bwd_lds<S56>(), a, st);
      break;
  }
  if (e != hipSuccess || (!a.want_dT && !a.want_dW)) return e;
  e = launch_bwd_reduce(a.partT, a.want_dW ? a.partW : nullptr, g, r.C, (int)L,
                        r.dT, a.want_dW ? r.dmixw : nullptr, st);
  if (e != hipSuccess || !a.want_dTs) return e;
  return launch_bwd_reduce(a.partTs, nullptr, g, r.C, (2 * r.s - 1) * (2 * r.s - 1), r.dTsub,
                           nullptr, st);
}

}  // namespace wbmm
