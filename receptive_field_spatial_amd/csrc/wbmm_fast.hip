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
#include "wbmm_fast.hpp"

#include <atomic>

namespace wbmm {

// ---------------------------------------------------------------------------- forward
// 12 waves: 8 consumers (2 per SIMD; consumer c contracts row tiles half c >> 2 of wave-unit
// c & 3) and 4 producers (wave-unit p). LDS: tables [2][TP] (by step parity; TP = LP, or 2 LP
// with the folded copy) and regions
// [3][4][RSZ] (unit k in k % 3). Step k:
//   consumers: contract unit k | barrier | accumulators -> region (z over X) | barrier
//   producers: issue loads of unit k+1, epilogue (mix, stores) of unit k-1 | barrier |
//              commit the loads | barrier
// The mid-step barrier keeps a half from overwriting X while the other half still reads it.

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

  float zpre[BwdCol<S>::NP][S::IH];
  {
    PlaneLoad<S> pl;
    pl.issue(a.dy + U.base, U, ir0, lane);
    // Issue order dy, table, z (z only feeds the dWmix sums). Loads complete in issue order for
    // the wait counter, so the table's LDS writes and the dy commit wait for dy and the table
    // only, and z lands during the sweep; the table's loads are clamped and unconditional, all
    // in flight before its writes.
    constexpr int TQ = (S::L + kThreads - 1) / kThreads;
    float tv[TQ], tsv[TQ];
#pragma unroll
    for (int j = 0; j < TQ; ++j) {
      const int q = threadIdx.x + j * kThreads, qc = q < S::L ? q : S::L - 1;
      tv[j] = a.T[(size_t)U.c * S::L + qc];
      if constexpr (HIER) tsv[j] = sub_entry<S>(a.Tsub, U.c, qc);
    }
    {
      // z, one register column per pass; unconditional (without dWmix these read dy, always
      // given, and go unused), so the wait for the table below is not widened at a branch merge
      const float* zu = (wantW ? a.zsaved : a.dy) + U.base;
#pragma unroll
      for (int p = 0; p < BwdCol<S>::NP; ++p) {
        const BwdCol<S> col(p, lane);
        const int ir = ir0 + col.im < U.nimg ? ir0 + col.im : U.nimg - 1;
        const int o = ir * U.cp + col.v;
#pragma unroll
        for (int h = 0; h < S::IH; ++h) zpre[p][h] = zu[o + h * S::IW];
      }
    }
    // unguarded writes (entries past the table land in its padding, which nothing reads), so
    // no load is sunk into a guard that would wait for every load in flight
    static_assert(S::LP > S::L, "table padding");
#pragma unroll
    for (int j = 0; j < TQ; ++j) {
      const int q = threadIdx.x + j * kThreads, qd = q < S::L ? q : S::L;
      Ts[qd] = tv[j];
      if constexpr (HIER) Ts[S::LP + qd] = tv[j] + tsv[j];
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
