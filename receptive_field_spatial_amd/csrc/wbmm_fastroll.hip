// Fast fp32 WBMM forward and backward on a window grid offset by half a window (w = 14, offsets
// 0 or 7, NCHW 14 x 14, 28 x 28 and 56 x 56 maps), through the rolled map.
#include "wbmm_fast.hpp"

namespace wbmm {

// ------------------------------------------------------------------- rolled offset grid
// The window grid offset by (oy, ox), each 0 or WS / 2, on IH x IW maps whose sides are multiples
// of WS [gecl.asia reading notes, "Limitation": windows interleaved between layers; pixels
// outside the map are zero, as for any ragged map]. Rolling the map by (-oy, -ox) moves every window of
// the offset grid, as whole quadrants at their own window positions, into one window of the plain
// grid of the rolled map: a plain window in the last window row (oy != 0) holds the lower half of
// an offset window above its upper half, and likewise for the last column, so a plain window
// holds one, two or four pieces. The product keeps the pairs of one piece: the matrix is masked
// to pairs whose quadrants agree on every split axis, and the pixels outside the map, zero in the
// offset grid, are simply not there. The work is then that of the plain grid (4 windows of a 28 x
// 28 map against 9 in the offset grid, 16 of a 56 x 56 map against 25).
//
// Unit = 16 images of one channel and 4 window positions (14 x 14 maps, one window per image: 64
// images), one workgroup of 4 waves; wave k holds window position k0 + k (row-major) of every
// image of the unit (14 x 14: the window of images 16k .. 16k + 15), image slot = MFMA column, so
// a wave's windows share one mask and the MFMA table operand stays one value per lane:
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

// A unit is 16 images of one channel and 4 window positions: all of a 28 x 28 map's, a quarter
// of a 56 x 56 map's (units per channel: ceil(B / 16) image groups x NWIN / 4 position groups,
// in a.groups); on 14 x 14 maps 64 images (ceil(B / 64) per channel). k0: the unit's first window
// position.
template <class S>
constexpr int roll_imgs() { return S::NWIN == 1 ? 64 : 16; }
template <class S>
__device__ __forceinline__ Unit roll_unit(const FastArgs& a, int u, int& k0) {
  constexpr int NPG = S::NWIN == 1 ? 1 : S::NWIN / 4;
  static_assert(S::NWIN == 1 || S::NWIN % 4 == 0, "whole position groups");
  Unit U;
  U.c = u / a.groups;
  const int rem = u - U.c * a.groups, ig = rem / NPG;
  k0 = 4 * (rem - ig * NPG);
  const int uimg0 = roll_imgs<S>() * ig;
  U.base = ((size_t)uimg0 * a.C + U.c) * S::PLANE;
  U.cp = a.C * S::PLANE;
  const int left = a.B - uimg0;
  U.nimg = left < roll_imgs<S>() ? left : roll_imgs<S>();
  return U;
}
// Wave k's part of the unit: its images (a Unit of at most 16) and its window position.
template <class S>
__device__ __forceinline__ Unit roll_wave(const Unit& U, int k0, int wave, int& pos, int& img0) {
  Unit W = U;
  if constexpr (S::NWIN == 1) {
    img0 = 16 * wave;
    W.base = U.base + (size_t)img0 * U.cp;
    const int left = U.nimg - img0;
    W.nimg = left < 0 ? 0 : (left < 16 ? left : 16);
    pos = 0;
  } else {
    img0 = 0;
    pos = k0 + wave;
  }
  return W;
}
// Table-gradient chunk ci (4 windows): its first image within the unit and its window position.
// Its windows sit in region ci / 4 at slots 4 (ci % 4) .. + 3 either way.
template <class S>
__device__ __forceinline__ void roll_chunk(int k0, int ci, int& img0, int& pos) {
  if constexpr (S::NWIN == 1) {
    img0 = 4 * ci;
    pos = 0;
  } else {
    img0 = 4 * (ci & 3);
    pos = k0 + (ci >> 2);
  }
}
template <class S>
int roll_groups(int B) {
  return S::NWIN == 1 ? (B + 63) / 64 : (B + 15) / 16 * (S::NWIN / 4);
}
// whole images in one unit: the forward applies the 3 x 3 mix on chip
template <class S>
constexpr bool roll_staged() { return S::NWIN <= 4; }

typedef float f4a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef float f3a4 __attribute__((ext_vector_type(3), aligned(4)));
typedef float f2a4 __attribute__((ext_vector_type(2), aligned(4)));

// The 49 pixels of quadrant q of plain window k of image slot n (lane (n, q) = (lane % 16,
// lane / 16)), read from the map through the roll: 7 half-rows of QW pixels, each contiguous in
// the map (the roll moves whole quadrants), as a 16-byte and a 12-byte load. Images past the
// batch are zero. Pixel s of the quadrant is the lane's MFMA operand of K step s.
template <class S>
struct RollQuad {
  static_assert(S::QW == 7, "14 x 14 windows");
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

// The unit's pre-mix maps in LDS (map coordinates) -> y (3 x 3 mix, or a copy) and z_save.
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
  for (int col = threadIdx.x; col < roll_imgs<S>() * S::IW; col += kThreads) {
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
// (56 x 56 maps: the table and the zeros only; the products are stored straight from the
// accumulators and the mix runs as a pass of its own.)
template <class S>
constexpr int roll_fwd_floats() {
  return roll_staged<S>() ? S::LP + roll_imgs<S>() * S::PLANE : S::LP + (S::CMAX + 4) / 4 * 4;
}

template <class S, bool MIX>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 8)))
k_roll_fwd(FastArgs a) {
  extern __shared__ __attribute__((aligned(16))) float smem_f[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* Ts = smem_f;
  constexpr int ZOFF =
      roll_staged<S>() ? S::LP + roll_imgs<S>() * S::PLANE - (S::CMAX + 4) / 4 * 4 : S::LP;
  static_assert(ZOFF >= S::LP && (roll_staged<S>() || !MIX), "zeros after the table");
  int k0, pos, img0;
  const Unit U = roll_unit<S>(a, blockIdx.x, k0);
  const Unit W = roll_wave<S>(U, k0, wave, pos, img0);
  const RollGeo g = roll_geo<S>(a, pos);
  RollQuad<S> xq;
  xq.load(a.x + W.base, W, g, lane);
  for (int q = threadIdx.x; q < S::L; q += kThreads) Ts[q] = a.T[(size_t)U.c * S::L + q];
  for (int q = threadIdx.x; q <= S::CMAX; q += kThreads) Ts[ZOFF + q] = 0.f;
  __syncthreads();
  if constexpr (roll_staged<S>()) {
    // thirds of the row tiles (5, 4, 4), held until every wave is past the zeros
    float* Z = smem_f + S::LP;
    v4f acc0[5], acc1[4], acc2[4];
    contract_roll<S, false, ZOFF, 0, 5>(Ts, xq.v, lane, g.gm, acc0);
    contract_roll<S, false, ZOFF, 5, 4>(Ts, xq.v, lane, g.gm, acc1);
    contract_roll<S, false, ZOFF, 9, 4>(Ts, xq.v, lane, g.gm, acc2);
    __syncthreads();
    roll_stage<S, 0, 5>(Z + img0 * S::PLANE, g, acc0, lane);
    roll_stage<S, 5, 4>(Z + img0 * S::PLANE, g, acc1, lane);
    roll_stage<S, 9, 4>(Z + img0 * S::PLANE, g, acc2, lane);
    __syncthreads();
    roll_epilogue<S, MIX>(a, Z, U);
  } else {  // each third stored while the next is contracted
    {
      v4f acc[5];
      contract_roll<S, false, ZOFF, 0, 5>(Ts, xq.v, lane, g.gm, acc);
      roll_store<S, 0, 5>(a.y, a.zsave, W, g, acc, lane);
    }
    {
      v4f acc[4];
      contract_roll<S, false, ZOFF, 5, 4>(Ts, xq.v, lane, g.gm, acc);
      roll_store<S, 5, 4>(a.y, a.zsave, W, g, acc, lane);
    }
    {
      v4f acc[4];
      contract_roll<S, false, ZOFF, 9, 4>(Ts, xq.v, lane, g.gm, acc);
      roll_store<S, 9, 4>(a.y, a.zsave, W, g, acc, lane);
    }
  }
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
// walks the unit in 16 chunks of 4 windows of one position (roll_chunk), with the row pairs of one
// band only where the rows are split and the column mask applied when the class's chains are
// promoted.
template <class S>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 8)))
k_roll_bwd(FastArgs a) {
  extern __shared__ __attribute__((aligned(16))) float smem_f[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* Ts = smem_f;
  float* regions = smem_f + bwd_tsz<S, false>();
  float* R = regions + wave * S::RSZ;
  const int u = blockIdx.x;
  int k0, pos, img0;
  const Unit U = roll_unit<S>(a, u, k0);
  const Unit W = roll_wave<S>(U, k0, wave, pos, img0);
  const RollGeo g = roll_geo<S>(a, pos);
  // G of the wave's windows in registers; during dX the zeros of the masked operands sit at the
  // start of the regions, which take G (for the table gradient) only after dX
  constexpr int ZOFF = bwd_tsz<S, false>();
  static_assert(S::CMAX < S::RSZ, "zeros inside the first region");
  RollQuad<S> gq;
  gq.load(a.dy + W.base, W, g, lane);
  for (int q = threadIdx.x; q < S::L; q += kThreads) Ts[q] = a.T[(size_t)U.c * S::L + q];
  for (int q = threadIdx.x; q <= S::CMAX; q += kThreads) Ts[ZOFF + q] = 0.f;
  __syncthreads();

  if (a.want_dx) {  // thirds of the row tiles, as in the forward
    {
      v4f acc[5];
      contract_roll<S, true, ZOFF, 0, 5>(Ts, gq.v, lane, g.gm, acc);
      roll_store<S, 0, 5>(a.dx, nullptr, W, g, acc, lane);
    }
    {
      v4f acc[4];
      contract_roll<S, true, ZOFF, 5, 4>(Ts, gq.v, lane, g.gm, acc);
      roll_store<S, 5, 4>(a.dx, nullptr, W, g, acc, lane);
    }
    {
      v4f acc[4];
      contract_roll<S, true, ZOFF, 9, 4>(Ts, gq.v, lane, g.gm, acc);
      roll_store<S, 9, 4>(a.dx, nullptr, W, g, acc, lane);
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
      int cimg, cpos;
      roll_chunk<S>(k0, ci, cimg, cpos);
      const RollGeo cg = roll_geo<S>(a, cpos);
      const int cbase = cimg * U.cp;
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
      int cimg, cpos;
      roll_chunk<S>(k0, ci, cimg, cpos);
      const RollGeo cg = roll_geo<S>(a, cpos);
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

static_assert(lds_fits(roll_fwd_floats<S28>() * 4, 3) && lds_fits(bwd_lds<S28>(), 3) &&
                  lds_fits(roll_fwd_floats<S56>() * 4, 3) && lds_fits(bwd_lds<S56>(), 3) &&
                  lds_fits(roll_fwd_floats<S14>() * 4, 3) && lds_fits(bwd_lds<S14>(), 3),
              "three rolled-grid workgroups per CU");

namespace {
// One workgroup of 4 waves per unit.
template <class S, class Fn>
hipError_t launch_roll(Fn fn, int lds, FastArgs a, hipStream_t st) {
  a.groups = roll_groups<S>(a.B);
  hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  return launch_main(fn, dim3(a.C * a.groups), dim3(kThreads), lds, st, a);
}
}  // namespace

// The offset grid on the rolled map: fp32, w = 14, NCHW 14 x 14, 28 x 28 or 56 x 56, offsets 0 or
// 7 (not both 0).
static bool roll_shape_ok(int B, int C, int H, int W, int w, int layout, int oy, int ox) {
  return w == 14 && layout == 0 && H == W && (H == 14 || H == 28 || H == 56) &&
         (oy == 0 || oy == 7) &&
         (ox == 0 || ox == 7) && (oy != 0 || ox != 0) && B >= 1 && C >= 1 &&
         offsets_fit(C, H, W) &&
         (H != 14 || (size_t)64 * C * H * W < ((size_t)1 << 31));  // 64-image units: int offsets
}

bool fast_roll_forward_ok(const FwdRequest& r) {
  return !r.in_bf16 && !r.out_bf16 && r.T && !r.M && !r.Tsub && !r.flip &&
         roll_shape_ok(r.B, r.C, r.H, r.W, r.w, r.layout, r.oy, r.ox);
}

bool fast_roll_backward_ok(const BwdRequest& r) {
  return r.T && !r.M && !r.Tsub && roll_shape_ok(r.B, r.C, r.H, r.W, r.w, r.layout, r.oy, r.ox);
}

// 56 x 56 maps with the mix and no z_save: the pre-mix map between the product and the mix pass.
size_t fast_roll_forward_workspace(const FwdRequest& r) {
  return fast_roll_forward_ok(r) && r.H == 56 && r.mixw && !r.zsave
             ? (size_t)r.B * r.C * r.H * r.W * sizeof(float)
             : 0;
}

// The layer on the offset grid: y (the 3 x 3 mix applied on chip on 14 x 14 and 28 x 28 maps, as
// a pass of its own after the product on 56 x 56 ones) and z_save (the pre-mix map).
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
  if (r.H == 28)
    return r.mixw ? launch_roll<S28>(k_roll_fwd<S28, true>, roll_fwd_floats<S28>() * 4, a, st)
                  : launch_roll<S28>(k_roll_fwd<S28, false>, roll_fwd_floats<S28>() * 4, a, st);
  if (r.H == 14)
    return r.mixw ? launch_roll<S14>(k_roll_fwd<S14, true>, roll_fwd_floats<S14>() * 4, a, st)
                  : launch_roll<S14>(k_roll_fwd<S14, false>, roll_fwd_floats<S14>() * 4, a, st);
  if (!r.mixw) return launch_roll<S56>(k_roll_fwd<S56, false>, roll_fwd_floats<S56>() * 4, a, st);
  float* z = (float*)(r.zsave ? r.zsave : r.ws);
  a.mixw = nullptr;
  a.y = z;
  a.zsave = nullptr;
  hipError_t e = launch_roll<S56>(k_roll_fwd<S56, false>, roll_fwd_floats<S56>() * 4, a, st);
  if (e != hipSuccess) return e;
  return launch_mix_fwd_f32_route(z, r.mixw, (float*)r.y, r.B, r.C, r.H, r.W, st);
}

// Table-gradient partials of the rolled backward: one fp64 row of L per unit.
size_t fast_roll_backward_workspace(const BwdRequest& r) {
  if (!fast_roll_backward_ok(r)) return 0;
  const size_t L = (size_t)(2 * r.w - 1) * (2 * r.w - 1);
  const int g = r.H == 14 ? roll_groups<S14>(r.B)
                : r.H == 28 ? roll_groups<S28>(r.B) : roll_groups<S56>(r.B);
  return ((size_t)r.C * g * L * 8 + 255) / 256 * 256;
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
  hipError_t e = r.H == 14   ? launch_roll<S14>(k_roll_bwd<S14>, bwd_lds<S14>(), a, st)
                  : r.H == 28 ? launch_roll<S28>(k_roll_bwd<S28>, bwd_lds<S28>(), a, st)
                              : launch_roll<S56>(k_roll_bwd<S56>, bwd_lds<S56>(), a, st);
  if (e != hipSuccess || !a.want_dT) return e;
  const int L = (2 * r.w - 1) * (2 * r.w - 1);
  const int g = r.H == 14 ? roll_groups<S14>(r.B)
                : r.H == 28 ? roll_groups<S28>(r.B) : roll_groups<S56>(r.B);
  return launch_bwd_reduce(a.partT, nullptr, g, r.C, L, r.dT, nullptr, st);
}

}  // namespace wbmm
