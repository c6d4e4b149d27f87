// Fast fp32 WBMM forward from the relative-position table (w = 14, NCHW, any H and W), with an
// optional 7 x 7 sub-window table folded on chip: the padded, ragged maps of dense prediction
// [arxivdaily abstract: high-resolution dense prediction; gecl.asia reading notes, "Core Idea":
// M_c[i][j] = T_c[(y_i - y_j) + w - 1][(x_i - x_j) + w - 1]; "Method": the hierarchical fold adds
// the sub-window table on pairs of one 7 x 7 sub-window].
//
// Persistent waves, one workgroup of 8 per CU (two waves per SIMD). Every wave keeps its own copy
// of the current channel's table in LDS (stored reversed, so every A read is a per-lane base plus
// a non-negative immediate), and with the fold a second, folded copy Tf = T + T_sub on the central
// entries; waves never wait for each other. A window's 196 outputs are 13 row tiles of 16; the
// work list is (channel, wave-unit of 16 windows, third of the row tiles: 5, 4, 4 tiles), so that
// the chip's SIMDs get equal shares even when a map has few wave-units per SIMD. Per item:
//   * B operand (window pixels) straight from HBM into registers: lane (n, g) holds the 49 pixels
//     of quadrant g of window n, kept while a wave's items stay in one wave-unit; the other wave
//     of the SIMD computes while they load. Windows are listed whole ones first; quadrant rows
//     are read as a 16-byte and a 12-byte load, rows outside the map at an offset past the end
//     of the buffer, which the hardware answers with zero; wave-units with a quadrant cut by
//     the map's edge in columns read pixel by pixel;
//   * A operand M_c[m][k] for K step s of quadrant g: one LDS read of the (folded) reversed table at
//     the tile's lane base plus 27 (s / 7) + s % 7, two steps ahead of their MFMAs;
//   * v_mfma_f32_16x16x4f32, the third's tiles as independent chains over 49 K steps;
//   * outputs stored from the accumulators (reverse + crop fused) as pixel pairs, to y or the
//     pre-mix map; stores of padding rows and of pixels outside the map go past the end of the
//     buffer and are dropped.
#include "wbmm_device.hpp"
#include "wbmm_launch.hpp"

#include <algorithm>
#include <atomic>

namespace wbmm {
namespace {

constexpr int TW = 14, TD = TW * TW, TQ = 7, TKQ = TQ * TQ;  // window, pixels, quadrant side, steps
constexpr int TRT = (TD + 15) / 16;                          // row tiles, 13
constexpr int TL1 = 2 * TW - 1, TL = TL1 * TL1;              // 27, 729
constexpr int SL1 = 2 * TQ - 1;                              // sub-table side, 13
constexpr int kTabPerSimd = 2;  // waves per SIMD (1: 33.5 us, 3: 31.1 us against 29.9 on the
                                // 2 x 128 x 128^2 map)
constexpr int kTabWaves = 4 * kTabPerSimd, kTabThreads = kTabWaves * 64;
constexpr int TPITCH = 736;                                  // floats per table copy
// LDS requested per workgroup: more than half a CU's 160 KB, so one workgroup per CU (the
// waves' tables use 23.5 KB of it)
constexpr int kTabLdsReserve = 96 * 1024;
// An offset at or past every buffer this kernel reads (x is below kTabOob bytes); two of them
// still sum below 2^32.
constexpr int kTabOob = 0x7fff0000;
static_assert(kTabWaves * 2 * TPITCH * 4 <= kTabLdsReserve, "per-wave tables fit");

struct TabArgs {
  int B, C, H, W;
  int oy, ox;        // window grid offset: window (wy, wx) starts at map pixel (14 wy - oy, 14 wx - ox)
  int nWx, nWy, nWin;  // windows per image row, per image column, per image
  int ix0, iy0;      // first whole window column, row
  int nIx, nIy;      // whole windows per image row, per image column
  int nIn;           // whole windows per image (nIx * nIy)
  int wupc;          // wave-units per channel: ceil(B * nWin / 16)
  long long items;   // C * wupc * 3
  int nsimd;         // SIMD ranges sharing the items (kTabPerSimd waves each)
  const float* x;
  const float* T;    // (C, 27, 27)
  const float* Ts;   // (C, 13, 13) folded on chip, or null
  float* out;        // y, or the pre-mix map when the mix runs as its own pass
  float* out2;       // z_save written with the same values (no mix), or null
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tab_x_rsrc(const TabArgs& a) {
  const long long bytes = (long long)a.B * a.C * a.H * a.W * 4;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.x), (short)0, (int)bytes,
                                           0x00020000);
}

// Window order within a channel: the whole windows of every image first (image by image,
// row-major over the whole-window block), then the partial ones at the map border (per image,
// row-major over the frame around that block), so that most wave-units hold only whole windows
// and take the vector loads below.
__device__ __forceinline__ void tab_window(const TabArgs& a, int win, int& b, int& wy, int& wx) {
  const int nin_all = a.B * a.nIn;
  if (win < nin_all) {
    b = win / a.nIn;
    const int i = win - b * a.nIn;
    const int ry = i / a.nIx;
    wy = a.iy0 + ry;
    wx = a.ix0 + (i - ry * a.nIx);
  } else {
    const int nbd = a.nWin - a.nIn, j = win - nin_all;
    b = j / nbd;
    const int i = j - b * nbd;
    const int top = a.iy0 * a.nWx, per = a.nWx - a.nIx, mid = a.nIy * per;
    if (i < top) {  // rows above the whole-window block
      wy = i / a.nWx;
      wx = i - wy * a.nWx;
    } else if (i < top + mid) {  // the block's rows: columns left and right of it
      const int k = i - top, ry = k / per, e = k - ry * per;
      wy = a.iy0 + ry;
      wx = e < a.ix0 ? e : e + a.nIx;
    } else {  // rows below it
      const int k = i - top - mid, ry = k / a.nWx;
      wy = a.iy0 + a.nIy + ry;
      wx = k - ry * a.nWx;
    }
  }
}

typedef float tab_f3 __attribute__((ext_vector_type(3)));
typedef float tab_f4 __attribute__((ext_vector_type(4)));

// The 49 pixels of quadrant g of the lane's window (zeros outside the map and past the last
// window), pixel s at quadrant row s / 7, column s % 7.
// The lane's window coordinates and output origin ride along for the stores.
struct TabXLoad {
  float v[TKQ];
  long long wbase;   // element offset of the window's origin in the map (negative above or left
                     // of a plane's origin on an offset grid: only its in-map pixels are used)
  int wy, wx;        // window row and column
  bool valid;        // a window of the batch (not past the last one)
  bool whole;        // the window lies inside the map
  __device__ __forceinline__ void issue(const TabArgs& a, __amdgpu_buffer_rsrc_t xr, int c,
                                        int win, int g) {
    const int nwin_ch = a.B * a.nWin;
    valid = win < nwin_ch;
    int b;
    tab_window(a, valid ? win : 0, b, wy, wx);
    const int y0 = wy * TW - a.oy, x0 = wx * TW - a.ox;  // map pixel of the window origin
    wbase = ((long long)b * a.C + c) * a.H * a.W + (long long)y0 * a.W + x0;
    whole = y0 >= 0 && x0 >= 0 && y0 + TW <= a.H && x0 + TW <= a.W;
    const int r0 = y0 + TQ * (g >> 1), c0 = x0 + TQ * (g & 1);
    const int vo = (int)((wbase + (long long)(TQ * (g >> 1)) * a.W + TQ * (g & 1)) * 4);
    const int rowb = a.W * 4;
    // A quadrant whose columns lie all inside or all outside the map reads its rows as a
    // 16-byte and a 12-byte load (4-byte aligned); rows outside the map, and every row of a
    // quadrant outside in columns, take an offset past the end of the buffer and read zeros.
    // (Quadrants of an offset grid are of this kind when the column offset is 0 or 7; a map
    // whose width is no multiple of 7 has quadrants cut by its right edge.)
    const bool cols_in = c0 >= 0 && c0 + TQ <= a.W, cols_out = c0 + TQ <= 0 || c0 >= a.W;
    const bool cut = valid && !cols_in && !cols_out;
    if (__builtin_amdgcn_ballot_w64(cut) == 0) {
#pragma unroll
      for (int r = 0; r < TQ; ++r) {
        const bool rok = valid && cols_in && r0 + r >= 0 && r0 + r < a.H;
        const int ro = rok ? vo + r * rowb : kTabOob;
        // (the loads' integer vectors are cast whole: this compiler narrows a component read of
        // them to a one-dword load)
        const tab_f4 p = __builtin_bit_cast(tab_f4, __builtin_amdgcn_raw_buffer_load_b128(xr, ro, 0, 0));
        const tab_f3 q =
            __builtin_bit_cast(tab_f3, __builtin_amdgcn_raw_buffer_load_b96(xr, ro + 16, 0, 0));
        v[TQ * r + 0] = p.x;
        v[TQ * r + 1] = p.y;
        v[TQ * r + 2] = p.z;
        v[TQ * r + 3] = p.w;
        v[TQ * r + 4] = q.x;
        v[TQ * r + 5] = q.y;
        v[TQ * r + 6] = q.z;
      }
    } else {
      // pixel by pixel: pixels outside the map get a row or column offset of kTabOob, which
      // puts the sum past the buffer's end: the hardware returns zero, so no select waits on
      // the loads
      int rowo[TQ], colo[TQ];
#pragma unroll
      for (int r = 0; r < TQ; ++r)
        rowo[r] = valid && r0 + r >= 0 && r0 + r < a.H ? vo + r * rowb : kTabOob;
#pragma unroll
      for (int q = 0; q < TQ; ++q) colo[q] = c0 + q >= 0 && c0 + q < a.W ? q * 4 : kTabOob;
#pragma unroll
      for (int s = 0; s < TKQ; ++s)
        v[s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                             xr, rowo[s / TQ] + colo[s % TQ], 0, 0));
    }
  }
};

// Reversed-table offset of K step s (pixel s of the lane's quadrant) from the lane's tile base.
__device__ __forceinline__ constexpr int kstep_off(int s) { return TL1 * (s / TQ) + s % TQ; }

// Per-lane constants of the 13 row tiles, formed once per wave: the lane's base in the reversed
// table (the folded copy when row m and the lane's quadrant g are one sub-window), and the map
// byte offsets, relative to the window origin, of its output pixels p0 = 16 t + 4 g and p0 + 2
// (kTabOob for the padding lanes of tile 12; a window origin plus kTabOob stays below 2^32).
struct TabLane {
  int rb[TRT], po[TRT], po2[TRT];
  template <bool HIER>
  __device__ __forceinline__ void init(int n, int g, int W) {
#pragma unroll
    for (int t = 0; t < TRT; ++t) {
      const int m = min(16 * t + n, TD - 1);  // rows past 195 repeat row 195, unused
      const int ym = m / TW, xm = m - (m / TW) * TW;
      const int base = (ym - TQ * (g >> 1) + TW - 1) * TL1 + (xm - TQ * (g & 1) + TW - 1);
      int off = TL - 1 - base;
      if (HIER && ym / TQ == (g >> 1) && xm / TQ == (g & 1)) off += TPITCH;
      rb[t] = off;
      const int p0 = 16 * t + 4 * g;
      po[t] = p0 < TD ? 4 * ((p0 / TW) * W + p0 % TW) : kTabOob;
      po2[t] = p0 < TD ? 4 * (((p0 + 2) / TW) * W + (p0 + 2) % TW) : kTabOob;
    }
  }
};

// The tiles [T0, T0 + NT) of one wave-unit: accumulate, then store.
template <bool HIER, int T0, int NT>
__device__ __forceinline__ void tab_contract(const TabArgs& a, const float* Tw, const TabXLoad& xl,
                                             const TabLane& tl, __amdgpu_buffer_rsrc_t yr,
                                             __amdgpu_buffer_rsrc_t y2r, int g) {
  const float(&xv)[TKQ] = xl.v;
  int rb[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) rb[i] = tl.rb[T0 + i];
  v4f acc[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
  // A values two K steps ahead of their MFMAs
  float a0[NT], a1[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    a0[i] = Tw[rb[i] + kstep_off(0)];
    a1[i] = Tw[rb[i] + kstep_off(1)];
  }
#pragma unroll
  for (int s = 0; s < TKQ; s += 2) {
    float b0[NT], b1[NT];
    if (s + 2 < TKQ) {
#pragma unroll
      for (int i = 0; i < NT; ++i) b0[i] = Tw[rb[i] + kstep_off(s + 2)];
    }
    if (s + 3 < TKQ) {
#pragma unroll
      for (int i = 0; i < NT; ++i) b1[i] = Tw[rb[i] + kstep_off(s + 3)];
    }
    __builtin_amdgcn_sched_barrier(0);  // the reads go out before this pair's MFMAs
#pragma unroll
    for (int i = 0; i < NT; ++i) acc[i] = mfma_f32(a0[i], xv[s], acc[i]);
    if (s + 1 < TKQ) {
#pragma unroll
      for (int i = 0; i < NT; ++i) acc[i] = mfma_f32(a1[i], xv[s + 1], acc[i]);
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      a0[i] = b0[i];
      a1[i] = b1[i];
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // reverse + crop: lane (n, g) holds pixels 16 t + 4 g .. + 3 of its window. Buffer stores
  // at 32-bit offsets; an offset of kTabOob (past the end) drops a store, which covers the
  // padding rows of tile 12 and, in border windows, the pixels outside the map.
  const bool valid = xl.valid, whole = xl.whole;
  // byte offset of the window origin, modulo 2^32: the offset of every in-map pixel from it is
  // exact (the map is < 2^31 bytes)
  const unsigned ob = (unsigned)(unsigned long long)xl.wbase * 4u;
  // the window rows [rlo, rhi) and columns [clo, chi) that lie in the map
  const int y0 = xl.wy * TW - a.oy, x0 = xl.wx * TW - a.ox;
  const int rlo = -y0, rhi = a.H - y0, clo = -x0, chi = a.W - x0;
  if (!valid) return;
  typedef uint32_t tab_u2 __attribute__((ext_vector_type(2)));
  auto put2 = [&](unsigned off, float v0, float v1) {
    const tab_u2 d = __builtin_bit_cast(tab_u2, make_float2(v0, v1));
    __builtin_amdgcn_raw_buffer_store_b64(d, yr, (int)off, 0, 0);
    if (a.out2) __builtin_amdgcn_raw_buffer_store_b64(d, y2r, (int)off, 0, 0);
  };
  auto put1 = [&](unsigned off, float v0) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v0), yr, (int)off, 0, 0);
    if (a.out2)
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v0), y2r, (int)off, 0, 0);
  };
  if (whole) {
    // pixels p0, p0 + 1 share a window row (p0 is even, column <= 12); p0 + 2, p0 + 3 too
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const v4f v = acc[i];
      put2(ob + (unsigned)tl.po[T0 + i], v[0], v[1]);
      put2(ob + (unsigned)tl.po2[T0 + i], v[2], v[3]);
    }
  } else if (((a.W | a.ox) & 1) == 0) {
    // a border window, map width and column offset even: a pixel pair (even map column first)
    // is inside or outside as a whole
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int p0 = 16 * (T0 + i) + 4 * g, p2 = p0 + 2;
      const bool in0 = p0 < TD && p0 / TW >= rlo && p0 / TW < rhi && p0 % TW >= clo && p0 % TW < chi;
      const bool in2 = p0 < TD && p2 / TW >= rlo && p2 / TW < rhi && p2 % TW >= clo && p2 % TW < chi;
      const v4f v = acc[i];
      put2(in0 ? ob + (unsigned)tl.po[T0 + i] : (unsigned)kTabOob, v[0], v[1]);
      put2(in2 ? ob + (unsigned)tl.po2[T0 + i] : (unsigned)kTabOob, v[2], v[3]);
    }
  } else {  // a border window otherwise: pixel by pixel, inside the map only
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = 16 * (T0 + i) + 4 * g + r;
        const bool in = p < TD && p / TW >= rlo && p / TW < rhi && p % TW >= clo && p % TW < chi;
        put1(in ? ob + 4u * (unsigned)((p / TW) * a.W + p % TW) : (unsigned)kTabOob, acc[i][r]);
      }
  }
}

template <bool HIER>
__global__ void __launch_bounds__(kTabThreads) k_fwd_tab(TabArgs a) {
  extern __shared__ __attribute__((aligned(16))) float smem_f[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  float* Tw = smem_f + wave * 2 * TPITCH;
  // The waves on one SIMD (waves w, w + 4, ...) share a contiguous range of items and take
  // alternate items of it, so SIMDs get equal shares and one wave's loads wait while another
  // wave's MFMAs run.
  const long long sid = (long long)blockIdx.x * 4 + (wave & 3);
  const int slot = wave >> 2;
  if (sid >= a.nsimd) return;  // uniform over the wave
  const long long lo = a.items * sid / a.nsimd, hi = a.items * (sid + 1) / a.nsimd;

  const __amdgpu_buffer_rsrc_t xr = tab_x_rsrc(a);
  const int map_bytes = (int)((long long)a.B * a.C * a.H * a.W * 4);
  const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(a.out, (short)0, map_bytes,
                                                                      0x00020000);
  const __amdgpu_buffer_rsrc_t y2r = __builtin_amdgcn_make_buffer_rsrc(
      a.out2 ? a.out2 : a.out, (short)0, map_bytes, 0x00020000);
  // The channel's table (reversed) and the folded copy (T + T_sub where |dy|, |dx| < 7): the
  // loads go out before the next wave-unit's pixel loads, so waiting for them does not wait
  // for those.
  constexpr int NE = (TL + 63) / 64;  // 12 entries per lane
  float tv[NE], sv[NE];
  auto stage_load = [&](int c) {
    const float* src = a.T + (size_t)c * TL;
    const float* sub = HIER ? a.Ts + (size_t)c * SL1 * SL1 : nullptr;
#pragma unroll
    for (int j = 0; j < NE; ++j) {
      const int e = min(lane + 64 * j, TL - 1);
      tv[j] = src[e];
      if constexpr (HIER) {
        const int dy = e / TL1 - (TW - 1), dx = e % TL1 - (TW - 1);
        const bool central = dy > -TQ && dy < TQ && dx > -TQ && dx < TQ;
        sv[j] = sub[central ? (dy + TQ - 1) * SL1 + dx + TQ - 1 : 0];
      }
    }
  };
  auto stage_write = [&]() {
    __builtin_amdgcn_wave_barrier();  // the previous channel's reads are issued before these
#pragma unroll
    for (int j = 0; j < NE; ++j) {
      const int e = lane + 64 * j;
      if (e < TL) {
        Tw[TL - 1 - e] = tv[j];
        if constexpr (HIER) {
          const int dy = e / TL1 - (TW - 1), dx = e % TL1 - (TW - 1);
          const bool central = dy > -TQ && dy < TQ && dx > -TQ && dx < TQ;
          Tw[TPITCH + TL - 1 - e] = central ? tv[j] + sv[j] : tv[j];
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  TabLane tl;
  tl.init<HIER>(n, g, a.W);
  int staged = -1;
  long long loaded = -1;
  TabXLoad xl;
  for (long long it = lo + slot; it < hi; it += kTabPerSimd) {
    const long long u = it / 3;
    const int h = (int)(it - 3 * u);
    const int c = (int)(u / a.wupc), k = (int)(u - (long long)c * a.wupc);
    const bool restage = c != staged, reload = u != loaded;  // uniform
    if (restage) stage_load(c);
    __builtin_amdgcn_sched_barrier(0);
    if (reload) {
      xl.issue(a, xr, c, 16 * k + n, g);
      loaded = u;
    }
    __builtin_amdgcn_sched_barrier(0);
    if (restage) {
      stage_write();
      staged = c;
    }
    // the lane's quadrant passes through an empty asm, so that what the border stores derive
    // from it is formed per item instead of being hoisted out of the loop for all 13 tiles
    int g2 = g;
    asm volatile("" : "+v"(g2));
    if (h == 0) tab_contract<HIER, 0, 5>(a, Tw, xl, tl, yr, y2r, g2);
    else if (h == 1) tab_contract<HIER, 5, 4>(a, Tw, xl, tl, yr, y2r, g2);
    else tab_contract<HIER, 9, 4>(a, Tw, xl, tl, yr, y2r, g2);
  }
}

int tab_cu_count() {
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

}  // namespace

bool fast_tab_forward_ok(const FwdRequest& r) {
  return !r.in_bf16 && !r.out_bf16 && r.T && !r.M && r.w == TW && r.layout == 0 && r.oy >= 0 &&
         r.oy < TW && r.ox >= 0 && r.ox < TW && (!r.Tsub || r.s == TQ) && r.B >= 1 && r.C >= 1 &&
         (long long)r.B * r.C * r.H * r.W * 4 < kTabOob - (1 << 16);
}

// out: where the contraction's result goes (y, or the pre-mix map); out2: a second copy or null.
hipError_t launch_forward_fast_tab(const FwdRequest& r, float* out, float* out2, hipStream_t st) {
  TabArgs a{};
  a.B = r.B;
  a.C = r.C;
  a.H = r.H;
  a.W = r.W;
  a.oy = r.oy;
  a.ox = r.ox;
  a.nWx = (r.W + r.ox + TW - 1) / TW;
  a.nWy = (r.H + r.oy + TW - 1) / TW;
  a.nWin = a.nWx * a.nWy;
  a.ix0 = (r.ox + TW - 1) / TW;  // 1 when the grid is offset, else 0
  a.iy0 = (r.oy + TW - 1) / TW;
  a.nIx = std::max(0, (r.W + r.ox) / TW - a.ix0);
  a.nIy = std::max(0, (r.H + r.oy) / TW - a.iy0);
  a.nIn = a.nIx * a.nIy;
  a.wupc = (int)(((long long)r.B * a.nWin + 15) / 16);
  a.items = (long long)r.C * a.wupc * 3;
  a.x = (const float*)r.x;
  a.T = (const float*)r.T;
  a.Ts = r.Tsub;
  a.out = out;
  a.out2 = out2;
  const long long cap = 4LL * tab_cu_count();
  a.nsimd = (int)(a.items < cap ? a.items : cap);
  const int grid = (a.nsimd + 3) / 4;
  if (r.Tsub)
    return launch_main(k_fwd_tab<true>, dim3(grid), dim3(kTabThreads), kTabLdsReserve, st, a);
  return launch_main(k_fwd_tab<false>, dim3(grid), dim3(kTabThreads), kTabLdsReserve, st, a);
}

}  // namespace wbmm
