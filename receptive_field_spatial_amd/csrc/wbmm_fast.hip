// Fast fp32 WBMM forward and backward for compile-time shapes: window WS (even), image IH x IW
// (multiples of WS) in NCHW, with the images small enough that whole images fill one wave's 16
// MFMA columns (nWin = (IH/WS)(IW/WS) divides 16).
//
// Layout and dataflow (one workgroup = 4 waves = 64 windows of one channel):
//   * the table T_c sits in LDS once per workgroup; M_c is never formed: each MFMA A operand is
//     one table entry picked by the pair's relative offset [gecl.asia reading notes, "Core Idea";
//     the notes' "Limitation"/"Takeaway" name such a non-materializing kernel as future work];
//   * each wave keeps its 16 windows in its own LDS region, window-major (a window's WS*WS pixels
//     contiguous, row-major) — one contiguous block per window [pith page, Fig. 2 caption];
//   * K (the WS*WS pixels of a window) is walked as four (WS/2)x(WS/2) quadrants, one per MFMA
//     lane group, so for every K-step the table offset splits into a per-lane base plus a
//     compile-time constant: every A operand is one LDS read with an immediate offset;
//   * B operands (window pixels) stay in registers for the whole contraction;
//   * 3x3 mixes walk image columns with a sliding 3x3 register window (3 LDS reads per pixel).
#include "wbmm_core.hpp"
#include "wbmm_launch.hpp"

namespace wbmm {

struct FastArgs {
  int B, C;
  int wgs_per_c;
  const float* x;       // forward: x; backward: x
  const float* T;
  const float* mixw;
  const float* zsaved;  // backward only
  const float* dy;      // backward only
  float* zsave;         // forward only
  float* y;             // forward only
  float* dx;
  float* dT;
  float* dmixw;
  double* partT;
  double* partW;
  int want_dx, want_dT, want_dW;
};

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
  static constexpr int XP = (D + 15) / 32 * 32 + 16;  // X-chunk window pitch: lane groups on disjoint banks
  static constexpr int TSZ = ((L + 3) / 4 * 4) > 4 * XP ? ((L + 3) / 4 * 4) : 4 * XP;  // table, later X chunks
  static constexpr int NWY = IH / WS, NWX = IW / WS, NWIN = NWY * NWX;
  static constexpr int IPW = 16 / NWIN;        // images per wave
  static constexpr int WPITCH = D;             // floats per window in LDS
  static constexpr int RSZ = 16 * WPITCH;      // floats per wave region
  static constexpr int PLANE = IH * IW;
  static constexpr int CMAX = (QW - 1) * L1 + (QW - 1);  // largest in-quadrant table offset
  static_assert(WS % 2 == 0 && IH % WS == 0 && IW % WS == 0 && 16 % NWIN == 0, "shape");
  static constexpr int COLS = IPW * IW;                   // image columns per wave
  static constexpr int CHUNK_IMGS = IW <= 64 ? (64 / IW < IPW ? 64 / IW : IPW) : 1;
  static constexpr int CHUNK_COLS = CHUNK_IMGS * IW;      // columns per pass (image aligned)
  static_assert(IW <= 64, "image width");
};

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

// Global image planes (NCHW, channel c) of the wave's images -> window-major LDS region.
template <class S>
__device__ __forceinline__ void load_region(const float* __restrict__ src, int B, int C, int c,
                                            int img0, float* R, int lane) {
#pragma unroll
  for (int c0 = 0; c0 < S::COLS; c0 += 64) {
    const int col = c0 + lane;
    if (col < S::COLS) {
      const int im = col / S::IW, v = col % S::IW;
      const int b = img0 + im;
      float* dst = R + col_part<S>(im, v);
      if (b < B) {
        const float* p = src + ((size_t)b * C + c) * S::PLANE + v;
#pragma unroll
        for (int h = 0; h < S::IH; ++h) dst[row_part<S>(h)] = p[h * S::IW];
      } else {
#pragma unroll
        for (int h = 0; h < S::IH; ++h) dst[row_part<S>(h)] = 0.f;
      }
    }
  }
}

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

// acc[t] = sum_s A[16t + lane%16][k(gq, s)] * B[k(gq, s)][n] with A from the table in LDS and B
// from the wave's region (window n = lane % 16); both are single LDS reads with immediate offsets.
// Non-flipped A entry: base(i) - (qoff + ktab(s)); flipped (M^T): L-1-base(i) + qoff + ktab(s).
template <class S, bool FLIP>
__device__ __forceinline__ void contract(const float* Ts, const float* R, int lane,
                                         v4f (&acc)[S::RT]) {
  const LaneGeo<S> lg(lane);
  const float* bsrc = R + lg.qbase();
  const float* abase[S::RT];
#pragma unroll
  for (int t = 0; t < S::RT; ++t) {
    int i = t * 16 + (lane & 15);
    if (i > S::D - 1) i = S::D - 1;
    const int base = (i / S::WS) * S::L1 + (i % S::WS) + S::C0;
    // non-flipped address = (base - qoff - CMAX) + (CMAX - ktab(s)), both parts >= 0
    abase[t] = FLIP ? Ts + (S::L - 1 - base + lg.qoff()) : Ts + (base - lg.qoff() - S::CMAX);
    acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int s = 0; s < S::KQ; ++s) {
    const float bv = bsrc[kpix<S>(s)];
#pragma unroll
    for (int t = 0; t < S::RT; ++t) {
      const float av = FLIP ? abase[t][ktab<S>(s)] : abase[t][S::CMAX - ktab<S>(s)];
      acc[t] = mfma_f32(av, bv, acc[t]);
    }
  }
}

// Accumulators back into the region at the pixel positions they belong to.
template <class S>
__device__ __forceinline__ void write_acc(float* R, int lane, const v4f (&acc)[S::RT]) {
  float* p = R + (lane & 15) * S::WPITCH + 4 * (lane >> 4);
#pragma unroll
  for (int t = 0; t < S::RT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (S::D % 16 != 0) {
        if (t * 16 + 4 * (lane >> 4) + r >= S::D) continue;
      }
      p[t * 16 + r] = acc[t][r];
    }
}

// Walk the wave's image columns; for every pixel call f(h, v_valid, center, 3x3 window w[u][t]
// = value at (h+u-1, v+t-1), zero outside the image, global element offset within the plane).
// Columns are processed in image-aligned passes so that neighbour columns are never in another
// pass. `f` may overwrite the pixel's own LDS slot with `write(value)` (rows above the current
// one are never read again).
template <class S, class F>
__device__ __forceinline__ void sweep_columns(float* R, int lane, F&& f) {
#pragma unroll
  for (int c0 = 0; c0 < S::COLS; c0 += S::CHUNK_COLS) {
    const bool active = lane < S::CHUNK_COLS && c0 + lane < S::COLS;
    const int col = active ? c0 + lane : c0;
    const int im = col / S::IW, v = col % S::IW;
    const bool hasL = v > 0, hasR = v + 1 < S::IW;
    float* pc = R + col_part<S>(im, v);
    const float* pl = R + col_part<S>(im, hasL ? v - 1 : v);
    const float* pr = R + col_part<S>(im, hasR ? v + 1 : v);
    float w[3][3];
    // rows -1 (zero) and 0
#pragma unroll
    for (int t = 0; t < 3; ++t) w[0][t] = 0.f;
    w[1][0] = hasL ? pl[row_part<S>(0)] : 0.f;
    w[1][1] = pc[row_part<S>(0)];
    w[1][2] = hasR ? pr[row_part<S>(0)] : 0.f;
#pragma unroll
    for (int h = 0; h < S::IH; ++h) {
      if (h + 1 < S::IH) {
        w[2][0] = hasL ? pl[row_part<S>(h + 1)] : 0.f;
        w[2][1] = pc[row_part<S>(h + 1)];
        w[2][2] = hasR ? pr[row_part<S>(h + 1)] : 0.f;
      } else {
        w[2][0] = w[2][1] = w[2][2] = 0.f;
      }
      if (active) f(im, h, v, w, pc + row_part<S>(h));
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        w[0][t] = w[1][t];
        w[1][t] = w[2][t];
      }
    }
  }
}

// ---------------------------------------------------------------------------- forward
template <class S>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 8))) k_fwd_fast(FastArgs a) {
  extern __shared__ __attribute__((aligned(16))) float smem_f[];
  const int c = blockIdx.y, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* Ts = smem_f;
  float* R = smem_f + S::TSZ + wave * S::RSZ;
  const int img0 = (blockIdx.x * 4 + wave) * S::IPW;

  for (int q = threadIdx.x; q < S::L; q += kThreads) Ts[q] = a.T[(size_t)c * S::L + q];
  load_region<S>(a.x, a.B, a.C, c, img0, R, lane);
  __syncthreads();

  v4f acc[S::RT];
  contract<S, false>(Ts, R, lane, acc);
  wave_sync_lds();
  write_acc<S>(R, lane, acc);
  wave_sync_lds();

  const bool mix = a.mixw != nullptr;
  float w9[9];
#pragma unroll
  for (int q = 0; q < 9; ++q) w9[q] = mix ? a.mixw[c * 9 + q] : 0.f;
  const int B = a.B, C = a.C;
  float* zs = a.zsave;
  float* yo = a.y;
  sweep_columns<S>(R, lane, [&](int im, int h, int v, const float (&w)[3][3], float*) {
    const int b = img0 + im;
    if (b >= B) return;
    const size_t off = ((size_t)b * C + c) * S::PLANE + h * S::IW + v;
    const float z = w[1][1];
    if (zs) zs[off] = z;
    float yv = z;
    if (mix) {
      yv = 0.f;
#pragma unroll
      for (int u = 0; u < 3; ++u)
#pragma unroll
        for (int t = 0; t < 3; ++t) yv = fmaf(w9[u * 3 + t], w[u][t], yv);
    }
    yo[off] = yv;
  });
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
template <class S, int Q>
__device__ __forceinline__ void dt_chunk(const float* regions, const float* xbuf, int n0, int kn,
                                         int xc, v4f (&a32)[8], double (&acc64)[8][4],
                                         bool flush) {
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
    if (y2 >= 0 && y2 < WS) a32[J] = mfma_f32(Av[y1], Bv[y2 < 0 ? 0 : (y2 < WS ? y2 : WS - 1)], a32[J]); \
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
    }
  }
}

template <class S, int Q>
__device__ __forceinline__ void dt_partial_write(double* scr, const double (&acc64)[8][4],
                                                 double* pT, int lane) {
  constexpr int WS = S::WS;
#define WBMM_DT_OUT(J)                                                                 \
  if constexpr (Slot<WS, Q, J>::valid) {                                               \
    _Pragma("unroll") for (int r = 0; r < 4; ++r)                                      \
        scr[(4 * (lane >> 4) + r) * 16 + (lane & 15)] = acc64[J][r];                   \
    wave_sync_lds();                                                                   \
    if (lane < S::L1) {                                                                \
      const int dxv = lane - (WS - 1);                                                 \
      double s = 0.0;                                                                  \
      for (int xa = 0; xa < WS; ++xa) {                                                \
        const int xb = xa - dxv;                                                       \
        if (xb >= 0 && xb < WS) s += scr[xa * 16 + xb];                                \
      }                                                                                \
      pT[(Slot<WS, Q, J>::dy + WS - 1) * S::L1 + lane] = s;                            \
    }                                                                                  \
    wave_sync_lds();                                                                   \
  }
  WBMM_DT_OUT(0) WBMM_DT_OUT(1) WBMM_DT_OUT(2) WBMM_DT_OUT(3)
  WBMM_DT_OUT(4) WBMM_DT_OUT(5) WBMM_DT_OUT(6) WBMM_DT_OUT(7)
#undef WBMM_DT_OUT
}

template <class S>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 8))) k_bwd_fast(FastArgs a) {
  extern __shared__ __attribute__((aligned(16))) float smem_f[];
  __shared__ double s_wred[4][9];
  const int c = blockIdx.y, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* Ts = smem_f;
  float* regions = smem_f + S::TSZ;
  float* R = regions + wave * S::RSZ;
  const int wg_img0 = blockIdx.x * 4 * S::IPW;
  const int img0 = wg_img0 + wave * S::IPW;
  const int B = a.B, C = a.C;
  const bool mix = a.mixw != nullptr;

  for (int q = threadIdx.x; q < S::L; q += kThreads) Ts[q] = a.T[(size_t)c * S::L + q];
  load_region<S>(a.dy, B, C, c, img0, R, lane);
  wave_sync_lds();

  // ---- G = partition(dz) in place; dz = mix adjoint of dy (correlation with rot180(W)).
  //      dWmix[u][t] = sum z[p][q] dy[p-u+1][q-t+1]: the same 3x3 dy window, times z.
  //      A sliding 3x3 register window walks each image column; the column's z values are
  //      loaded up front. Row h of dy is overwritten by G only after its last read.
  if (mix) {
    float w9[9];
#pragma unroll
    for (int q = 0; q < 9; ++q) w9[q] = a.mixw[(c * 9) + (8 - q)];  // rot180: W[2-u][2-t]
    const bool wantW = a.want_dW;
    double wacc[9];
#pragma unroll
    for (int q = 0; q < 9; ++q) wacc[q] = 0.0;
#pragma unroll
    for (int c0 = 0; c0 < S::COLS; c0 += S::CHUNK_COLS) {
      const bool active = lane < S::CHUNK_COLS && c0 + lane < S::COLS;
      const int col = active ? c0 + lane : c0;
      const int im = col / S::IW, v = col % S::IW;
      const int b = img0 + im;
      const bool real = active && b < B;
      const bool hasL = v > 0, hasR = v + 1 < S::IW;
      float* pc = R + col_part<S>(im, v);
      const float* pl = R + col_part<S>(im, hasL ? v - 1 : v);
      const float* pr = R + col_part<S>(im, hasR ? v + 1 : v);
      float zc[S::IH];
      if (wantW) {
        const float* zp = a.zsaved + ((size_t)(b < B ? b : B - 1) * C + c) * S::PLANE + v;
#pragma unroll
        for (int h = 0; h < S::IH; ++h) zc[h] = zp[h * S::IW];
      }
      float wcol[9];
#pragma unroll
      for (int q = 0; q < 9; ++q) wcol[q] = 0.f;
      float w[3][3];
#pragma unroll
      for (int t = 0; t < 3; ++t) w[0][t] = 0.f;
      w[1][0] = hasL ? pl[row_part<S>(0)] : 0.f;
      w[1][1] = pc[row_part<S>(0)];
      w[1][2] = hasR ? pr[row_part<S>(0)] : 0.f;
#pragma unroll
      for (int h = 0; h < S::IH; ++h) {
        if (h + 1 < S::IH) {
          w[2][0] = hasL ? pl[row_part<S>(h + 1)] : 0.f;
          w[2][1] = pc[row_part<S>(h + 1)];
          w[2][2] = hasR ? pr[row_part<S>(h + 1)] : 0.f;
        } else {
          w[2][0] = w[2][1] = w[2][2] = 0.f;
        }
        // w[u][t] = dy(h+u-1, v+t-1); dz(h,v) = sum_{u,t} W[2-u][2-t] w[u][t]
        float gsum = 0.f;
#pragma unroll
        for (int q = 0; q < 9; ++q) gsum = fmaf(w9[q], w[q / 3][q % 3], gsum);
        if (real) pc[row_part<S>(h)] = gsum;
        if (wantW) {
          const float z = real ? zc[h] : 0.f;
          // dWmix[u][t] += z * dy(h-u+1, v-t+1) = z * w[2-u][2-t]
#pragma unroll
          for (int q = 0; q < 9; ++q) wcol[q] = fmaf(z, w[2 - q / 3][2 - q % 3], wcol[q]);
        }
#pragma unroll
        for (int t = 0; t < 3; ++t) {
          w[0][t] = w[1][t];
          w[1][t] = w[2][t];
        }
      }
#pragma unroll
      for (int q = 0; q < 9; ++q) wacc[q] += (double)wcol[q];
    }
    if (wantW) {
#pragma unroll
      for (int q = 0; q < 9; ++q) {
        double v = wacc[q];
        for (int off = 32; off > 0; off >>= 1) v += __shfl_down(v, off, 64);
        if (lane == 0) s_wred[wave][q] = v;
      }
    }
  }
  __syncthreads();  // table, every wave's G and the dWmix wave sums are in LDS
  if (a.want_dW && threadIdx.x < 9) {
    const int q = threadIdx.x;
    a.partW[((size_t)c * a.wgs_per_c + blockIdx.x) * 9 + q] =
        ((s_wred[0][q] + s_wred[1][q]) + s_wred[2][q]) + s_wred[3][q];
  }

  // ---- dX = M^T . G, stored straight from the accumulators (G stays in LDS for dT)
  if (a.want_dx) {
    v4f acc[S::RT];
    contract<S, true>(Ts, R, lane, acc);
    const int n = lane & 15, i0 = 4 * (lane >> 4);
    const int im = n / S::NWIN, wi = n % S::NWIN;
    const int b = img0 + im;
    if (b < B) {
      float* o = a.dx + ((size_t)b * C + c) * S::PLANE + (wi / S::NWX) * S::WS * S::IW +
                 (wi % S::NWX) * S::WS;
#pragma unroll
      for (int t = 0; t < S::RT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = t * 16 + r + i0;
          if (i < S::D) {
            const int yy = i / S::WS, xx = i - yy * S::WS;
            o[yy * S::IW + xx] = acc[t][r];
          }
        }
    }
  }

  // ---- table gradient partial over the workgroup's 64 windows. X comes in chunks of 4 windows
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
    constexpr int CH_E = 4 * S::D;
    constexpr int EPT = (CH_E + kThreads - 1) / kThreads;
    int goff[EPT], loff[EPT], ekn[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int e = threadIdx.x + j * kThreads;
      const int ee = e < CH_E ? e : 0;
      ekn[j] = ee / S::D;
      const int p = ee % S::D;
      goff[j] = (p / S::WS) * S::IW + (p % S::WS);
      loff[j] = e < CH_E ? ekn[j] * S::XP + p : -1;
    }
    float stg[EPT];
    auto load_chunk = [&](int ci) {
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        const int n = 4 * ci + ekn[j];
        const int q = n >> 4, nl = n & 15;
        const int im = nl / S::NWIN, wi = nl % S::NWIN;
        int b = wg_img0 + q * S::IPW + im;
        b = b < B ? b : B - 1;  // windows past the batch have G = 0
        stg[j] = a.x[((size_t)b * C + c) * S::PLANE + (wi / S::NWX) * S::WS * S::IW +
                     (wi % S::NWX) * S::WS + goff[j]];
      }
    };
    const int kn = lane >> 4, x1 = lane & 15;
    const int xc = x1 < S::WS ? x1 : S::WS - 1;
    float* xbuf = Ts;
    load_chunk(0);
    __syncthreads();  // every wave is done with the table (dX)
    for (int ci = 0; ci < 16; ++ci) {
      if (ci > 0) __syncthreads();  // chunk ci-1 consumed by every wave
#pragma unroll
      for (int j = 0; j < EPT; ++j)
        if (loff[j] >= 0) xbuf[loff[j]] = stg[j];
      __syncthreads();
      if (ci + 1 < 16) load_chunk(ci + 1);
      const bool flush = (ci & 1) != 0;
      switch (wave) {
        case 0: dt_chunk<S, 0>(regions, xbuf, 4 * ci, kn, xc, a32, acc64, flush); break;
        case 1: dt_chunk<S, 1>(regions, xbuf, 4 * ci, kn, xc, a32, acc64, flush); break;
        case 2: dt_chunk<S, 2>(regions, xbuf, 4 * ci, kn, xc, a32, acc64, flush); break;
        default: dt_chunk<S, 3>(regions, xbuf, 4 * ci, kn, xc, a32, acc64, flush); break;
      }
    }
    double* pT = a.partT + ((size_t)c * a.wgs_per_c + blockIdx.x) * S::L;
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

template <class S>
int lds_bytes() { return (S::TSZ + 4 * S::RSZ) * 4; }

template <class S>
int wgs_per_c(int B) { return (B + 4 * S::IPW - 1) / (4 * S::IPW); }

template <class S, class Fn>
hipError_t launch_shape(Fn fn, FastArgs a, hipStream_t st) {
  a.wgs_per_c = wgs_per_c<S>(a.B);
  hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     lds_bytes<S>());
  if (e != hipSuccess) return e;
  mark_main_kernel(st, true);
  hipLaunchKernelGGL(fn, dim3(a.wgs_per_c, a.C, 1), dim3(kThreads), lds_bytes<S>(), st, a);
  e = hipGetLastError();
  mark_main_kernel(st, false);
  return e;
}

using S14 = Shape<14, 14, 14>;
using S28 = Shape<14, 28, 28>;
using S56 = Shape<14, 56, 56>;

}  // namespace

bool fast_forward_ok(const FwdRequest& r) {
  return !r.in_bf16 && !r.out_bf16 && r.T && !r.M &&
         fast_shape(r.H, r.W, r.w, r.layout) != FS_NONE;
}

bool fast_backward_ok(const BwdRequest& r) {
  return r.T && !r.M && fast_shape(r.H, r.W, r.w, r.layout) != FS_NONE;
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
  switch (fast_shape(r.H, r.W, r.w, r.layout)) {
    case FS_14_14_14: return launch_shape<S14>(k_fwd_fast<S14>, a, st);
    case FS_14_28_28: return launch_shape<S28>(k_fwd_fast<S28>, a, st);
    case FS_14_56_56: return launch_shape<S56>(k_fwd_fast<S56>, a, st);
    default: return hipErrorInvalidValue;
  }
}

size_t fast_backward_workspace(const BwdRequest& r) {
  int wgs;
  switch (fast_shape(r.H, r.W, r.w, r.layout)) {
    case FS_14_14_14: wgs = wgs_per_c<S14>(r.B); break;
    case FS_14_28_28: wgs = wgs_per_c<S28>(r.B); break;
    case FS_14_56_56: wgs = wgs_per_c<S56>(r.B); break;
    default: return 0;
  }
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  const size_t L = (size_t)(2 * r.w - 1) * (2 * r.w - 1);
  return al((size_t)r.C * wgs * L * 8) + al((size_t)r.C * wgs * 9 * 8);
}

hipError_t launch_backward_fast(const BwdRequest& r, hipStream_t st) {
  FastArgs a{};
  a.B = r.B;
  a.C = r.C;
  int wgs;
  const FastShape fs = fast_shape(r.H, r.W, r.w, r.layout);
  switch (fs) {
    case FS_14_14_14: wgs = wgs_per_c<S14>(r.B); break;
    case FS_14_28_28: wgs = wgs_per_c<S28>(r.B); break;
    case FS_14_56_56: wgs = wgs_per_c<S56>(r.B); break;
    default: return hipErrorInvalidValue;
  }
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  const size_t L = (size_t)(2 * r.w - 1) * (2 * r.w - 1);
  unsigned char* ws = (unsigned char*)r.ws;
  a.partT = (double*)ws;
  a.partW = (double*)(ws + al((size_t)r.C * wgs * L * 8));
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
  hipError_t e;
  switch (fs) {
    case FS_14_14_14: e = launch_shape<S14>(k_bwd_fast<S14>, a, st); break;
    case FS_14_28_28: e = launch_shape<S28>(k_bwd_fast<S28>, a, st); break;
    default: e = launch_shape<S56>(k_bwd_fast<S56>, a, st); break;
  }
  if (e != hipSuccess || (!a.want_dT && !a.want_dW)) return e;
  return launch_bwd_reduce(a.partT, a.want_dW ? a.partW : nullptr, wgs, r.C, (int)L,
                           a.want_dT ? r.dT : nullptr, a.want_dW ? r.dmixw : nullptr, st);
}

}  // namespace wbmm
