// Fast fp32 WBMM forward on a cached matrix (w = 14, NCHW, any H and W): the pages' inference
// caching, where the d x d matrices M_c are built once (and possibly folded) and then read from
// memory on every call [gecl.asia reading notes, "Method", last sentence; "Limitation" names
// materializing M as the memory cost of the method].
//
// One persistent workgroup of 8 waves per CU (two per SIMD: one wave's loads and stores overlap
// the other's matrix work). The workgroup holds one channel's whole matrix in
// LDS (196 rows at a pitch of 202 floats = 154.7 KB); each wave contracts a "wave-unit" of 16
// consecutive windows of that channel at a time (windows of a channel are numbered image by
// image, row-major), so the window pixels never pass through LDS:
//   * B operand (window pixels) straight from HBM into registers: lane (n, g) holds the 49 pixels
//     of quadrant g of window n, the next wave-unit's pixels in flight during the contraction;
//     the loads address x as one raw buffer (a 32-bit per-lane offset, the window row as a
//     uniform offset, the column as an immediate); pixels outside the map (the zero padding of
//     a map whose sides are not multiples of 14) are read at an offset past the end of the
//     buffer, which the hardware answers with zero;
//   * A operand (M_c[i][j]) from LDS, quadrant-major within each row (quadrant g's 49 columns at
//     offset 50 g), so two consecutive K-steps of a lane are one 8-byte read;
//   * v_mfma_f32_16x16x4f32: 13 row tiles x 49 K-steps per wave-unit;
//   * outputs stored from the accumulators (reverse + crop fused), to y or, with the 3x3 mix,
//     to the pre-mix map that a mix pass then reads.
// A workgroup walks a contiguous range of the (channel, wave-unit) list in rounds of 8
// wave-units of one channel; the matrix is restaged when the channel changes. With few channels
// of many wave-units each, every channel is split into equal parts instead, one workgroup (and one
// matrix staging) per part.
#include "wbmm_device.hpp"
#include "wbmm_launch.hpp"

#include <algorithm>
#include <atomic>

namespace wbmm {
namespace {

constexpr int kCmWaves = 8;  // two waves per SIMD
constexpr int kCmThreads = kCmWaves * 64;
constexpr int CW = 14, CD = CW * CW, CRT = (CD + 15) / 16;  // window, pixels, row tiles
constexpr int CQ = 7, CKQ = CQ * CQ;                        // quadrant side, K-steps
constexpr int SEGP = 50;                                    // LDS floats per quadrant segment
constexpr int MP = 4 * SEGP + 2;                            // LDS row pitch (floats)
constexpr int kCmLds = CD * MP * 4;  // the matrix
// An offset at or past the end of x (the host takes this path below kCmOob - 2^16 bytes); two of
// them still sum below 2^32.
constexpr int kCmOob = 0x7fff0000;
static_assert(kCmLds <= 160 * 1024, "one channel's matrix fits in LDS");

struct CmArgs {
  int B, C, H, W;
  int nWx, nWin;       // windows per image row, per image
  int wupc;            // wave-units per channel: ceil(B * nWin / 16)
  long long total;     // C * wupc
  int parts;           // > 0: workgroup rg takes part rg % parts of channel rg / parts
  const float* x;
  const float* M;      // (C, 196, 196)
  float* out;          // y, or the pre-mix map when the mix runs as its own pass
  float* out2;         // z_save written with the same values (no mix), or null
};

// Pixel s of quadrant g: window row 7 (g >> 1) + s / 7, column 7 (g & 1) + s % 7.
__device__ __forceinline__ int quad_col(int g, int s) {
  return (7 * (g >> 1) + s / 7) * CW + 7 * (g & 1) + s % 7;
}

// The x tensor as a raw buffer (the host takes this path only below 2^31 bytes): loads address it
// by a per-lane 32-bit byte offset, a uniform row offset and an immediate column offset.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t x_rsrc(const CmArgs& a) {
  const long long bytes = (long long)a.B * a.C * a.H * a.W * 4;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.x), (short)0, (int)bytes,
                                           0x00020000);
}

// The window pixels of one lane (window n of the wave-unit, quadrant g), 49 registers.
struct XLoad {
  float v[CKQ];
  // win: the lane's window index in the channel (>= B * nWin: no window, zeros)
  __device__ __forceinline__ void issue(const CmArgs& a, __amdgpu_buffer_rsrc_t xr, int c, int win,
                                        int g) {
    const int nwin_ch = a.B * a.nWin;
    const bool valid = win < nwin_ch;
    const int wn = valid ? win : 0;
    const int b = wn / a.nWin, wi = wn - b * a.nWin;
    const int wy = wi / a.nWx, wx = wi - wy * a.nWx;
    const int r0 = wy * CW + 7 * (g >> 1), c0 = wx * CW + 7 * (g & 1);
    // byte offset of the quadrant origin
    const int vo = (int)((((size_t)b * a.C + c) * a.H * a.W + (size_t)r0 * a.W + c0) * 4);
    const int rowb = a.W * 4;
    const bool inside = valid && r0 + 7 <= a.H && c0 + 7 <= a.W;
    if (__builtin_amdgcn_ballot_w64(!inside) == 0) {  // the whole wave is inside the map
#pragma unroll
      for (int s = 0; s < CKQ; ++s)
        v[s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                             xr, vo + (s % 7) * 4, (s / 7) * rowb, 0));
    } else {
      // rows / columns of the quadrant inside the map; out-of-map pixels take a row or column
      // offset of kCmOob, which puts the sum past the buffer's end: the hardware returns zero,
      // so no select waits on the loads
      const int nr = valid ? min(7, a.H - r0) : 0, nc = valid ? min(7, a.W - c0) : 0;
      int rowo[7], colo[7];
#pragma unroll
      for (int r = 0; r < 7; ++r) rowo[r] = r < nr ? vo + r * rowb : kCmOob;
#pragma unroll
      for (int q = 0; q < 7; ++q) colo[q] = q < nc ? q * 4 : kCmOob;
#pragma unroll
      for (int s = 0; s < CKQ; ++s)
        v[s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                             xr, rowo[s / 7] + colo[s % 7], 0, 0));
    }
  }
};

// LDS slot of matrix column j within a row: quadrant segment g(j), then the column's place in it.
__device__ __forceinline__ int col_slot(int j) {
  const int y = j / CW, xx = j - (j / CW) * CW;
  return ((y / 7) * 2 + xx / 7) * SEGP + (y % 7) * 7 + xx % 7;
}

// Stage M_c (row-major (196, 196) in HBM) into LDS: thread t < 245 moves the 16-byte pieces of
// column group cg = t % 49 (columns 4 cg .. 4 cg + 3, whose four LDS slots it computes once) in
// rows t / 49 + 5 m, eight pieces in flight before their LDS writes.
__device__ __forceinline__ void stage_matrix(const float* __restrict__ M, int c, float* Ms) {
  constexpr int NG = CD / 4, RS = kCmThreads / NG, NR = (CD + RS - 1) / RS;  // 49, 5, 40
  constexpr int KB = 8;
  const int t = threadIdx.x;
  if (t >= NG * RS) return;
  const int cg = t % NG, r0 = t / NG;
  int slot[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) slot[k] = col_slot(4 * cg + k);
  const float4* src = (const float4*)(M + (size_t)c * CD * CD) + cg;
#pragma unroll 1
  for (int m0 = 0; m0 < NR; m0 += KB) {
    float4 v[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int i = min(r0 + RS * (m0 + k), CD - 1);
      v[k] = src[i * NG];
    }
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int i = r0 + RS * (m0 + k);
      if (i < CD) {
        float* row = Ms + i * MP;
        row[slot[0]] = v[k].x;
        row[slot[1]] = v[k].y;
        row[slot[2]] = v[k].z;
        row[slot[3]] = v[k].w;
      }
    }
  }
}

__global__ void __launch_bounds__(kCmThreads) k_fwd_cm(CmArgs a) {
  extern __shared__ __attribute__((aligned(16))) float smem_f[];
  float* Ms = smem_f;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  // XCD-aware ranges: workgroups are dealt to the 8 XCDs round-robin (workgroup b runs on XCD
  // b % 8), so range r = (b % 8) (G / 8) + b / 8 gives each XCD a contiguous run of ranges; the
  // ranges that share a channel then mostly share an L2, and a matrix staged by one CU is read
  // from that L2 by its neighbours
  const int G = gridDim.x;
  const int rg = G % 8 == 0 ? (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
  long long lo, hi;
  if (a.parts > 0) {  // channel-aligned: each workgroup stages one matrix
    const int c = rg / a.parts, q = rg - c * a.parts;
    lo = (long long)c * a.wupc + (long long)a.wupc * q / a.parts;
    hi = (long long)c * a.wupc + (long long)a.wupc * (q + 1) / a.parts;
  } else {
    lo = a.total * rg / G;
    hi = a.total * (rg + 1) / G;
  }


  // A round is up to 8 consecutive wave-units of one channel, one per wave (waves past its end
  // idle); every wave walks the same rounds, so the barriers around a restage match.
  auto round_end = [&](long long r) {
    const long long cend = (r / a.wupc + 1) * (long long)a.wupc;
    return min(min(r + kCmWaves, cend), hi);
  };
  const __amdgpu_buffer_rsrc_t xr = x_rsrc(a);
  auto issue = [&](XLoad& xl, long long r, long long rend) {
    const long long wu = r + wave;
    if (r < hi && wu < rend) {
      const int c = (int)(wu / a.wupc), k = (int)(wu - (long long)c * a.wupc);
      xl.issue(a, xr, c, 16 * k + n, g);
    }
  };
  int staged = -1;
  XLoad cur;
  long long r0 = lo;
  long long rend = round_end(r0);
  issue(cur, r0, rend);
  while (r0 < hi) {
    const int c = (int)(r0 / a.wupc);
    if (c != staged) {
      __syncthreads();  // every wave is done with the previous channel's matrix
      stage_matrix(a.M, c, Ms);
      __syncthreads();
      staged = c;
    }
    const long long wu = r0 + wave;
    const bool mine = wu < rend;
    // the next round's wave-unit of this wave: its loads are in flight during the contraction
    const long long nr0 = rend;
    const long long nrend = nr0 < hi ? round_end(nr0) : hi;
    XLoad nxt;
    issue(nxt, nr0, nrend);
    if (mine) {
      // the lane's coordinates pass through an empty asm, so that the per-tile values derived
      // from them are formed per wave-unit instead of being held across the loop
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int n = ln & 15, g = ln >> 4;
      const float* abase = Ms + n * MP + g * SEGP;
      v4f acc[CRT];
#pragma unroll
      for (int t = 0; t < CRT; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
      // A operand: two K-steps per 8-byte LDS read; the next pair's reads are issued before the
      // current pair's 26 MFMAs, and scheduling barriers keep each pair's MFMAs together so that
      // the 13 independent accumulator chains interleave
      typedef float f2 __attribute__((ext_vector_type(2)));
      const float* arow[CRT];
#pragma unroll
      for (int t = 0; t < CRT; ++t)  // rows past 195 (tile 12, m >= 4) read row 195; their
        arow[t] = abase + (16 * t + n > CD - 1 ? CD - 1 - n : 16 * t) * MP;  // outputs are unused
      f2 ac[CRT];
#pragma unroll
      for (int t = 0; t < CRT; ++t) ac[t] = *(const f2*)(arow[t]);
#pragma unroll
      for (int s = 0; s < CKQ; s += 2) {
        f2 an[CRT];
        if (s + 2 < CKQ) {
#pragma unroll
          for (int t = 0; t < CRT; ++t) an[t] = *(const f2*)(arow[t] + s + 2);
        }
#pragma unroll
        for (int t = 0; t < CRT; ++t) acc[t] = mfma_f32(ac[t].x, cur.v[s], acc[t]);
        if (s + 1 < CKQ) {
#pragma unroll
          for (int t = 0; t < CRT; ++t) acc[t] = mfma_f32(ac[t].y, cur.v[s + 1], acc[t]);
        }
        if (s + 2 < CKQ) {
#pragma unroll
          for (int t = 0; t < CRT; ++t) ac[t] = an[t];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // reverse + crop: pixel p = 16 t + 4 g + r of window (b, wy, wx)
      const int k = (int)(wu - (long long)c * a.wupc);
      const int win = 16 * k + n;
      if (win < a.B * a.nWin) {
        const int b = win / a.nWin, wi = win - b * a.nWin;
        const int wy = wi / a.nWx, wx = wi - wy * a.nWx;
        const size_t wbase = ((size_t)b * a.C + c) * a.H * a.W + (size_t)(wy * CW) * a.W + wx * CW;
        const bool inside = wy * CW + CW <= a.H && wx * CW + CW <= a.W;
        float* o = a.out + wbase;
        float* o2 = a.out2 ? a.out2 + wbase : nullptr;
        if (inside) {
          // lane (n, g) holds pixels p0 .. p0 + 3 (p0 = 16 t + 4 g, even): one row run of four
          // (a 16-byte store at 4-byte alignment) unless p0 sits at column 12, where the run
          // wraps into the next window row (two 8-byte stores)
          typedef float f4u __attribute__((ext_vector_type(4), aligned(4)));
          typedef float f2u __attribute__((ext_vector_type(2), aligned(4)));
#pragma unroll
          for (int t = 0; t < CRT; ++t) {
            if (16 * t + 4 * g >= CD) continue;
            // pixel p0 = 16 t + 4 g of the window: its offset and window column
            const int p0 = 16 * t + 4 * g;
            const int ocol = p0 % CW, ooff = (p0 / CW) * a.W + ocol;
            const v4f v = acc[t];
            if (ocol <= CW - 4) {
              *(f4u*)(o + ooff) = f4u{v[0], v[1], v[2], v[3]};
              if (o2) *(f4u*)(o2 + ooff) = f4u{v[0], v[1], v[2], v[3]};
            } else {
              *(f2u*)(o + ooff) = f2u{v[0], v[1]};
              *(f2u*)(o + ooff + a.W - (CW - 2)) = f2u{v[2], v[3]};
              if (o2) {
                *(f2u*)(o2 + ooff) = f2u{v[0], v[1]};
                *(f2u*)(o2 + ooff + a.W - (CW - 2)) = f2u{v[2], v[3]};
              }
            }
          }
        } else {
          // a border window of a padded map: pixel by pixel, inside the map only
#pragma unroll
          for (int t = 0; t < CRT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int p = 16 * t + 4 * g + r;
              if (p >= CD) continue;
              const int py = wy * CW + p / CW, px = wx * CW + p % CW;
              if (py < a.H && px < a.W) {
                const int off = (p / CW) * a.W + p % CW;
                o[off] = acc[t][r];
                if (o2) o2[off] = acc[t][r];
              }
            }
        }
      }
    }
    cur = nxt;
    r0 = nr0;
    rend = nrend;
  }
}

int cm_cu_count() {
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

bool fast_cm_forward_ok(const FwdRequest& r) {
  return !r.in_bf16 && !r.out_bf16 && r.M && !r.T && !r.Tsub && r.w == CW && r.layout == 0 &&
         r.oy == 0 && r.ox == 0 && (long long)r.B * r.C * r.H * r.W * 4 < kCmOob - (1 << 16);
}

// out: where the contraction's result goes (y, or the pre-mix map); out2: a second copy or null.
hipError_t launch_forward_fast_cm(const FwdRequest& r, float* out, float* out2, hipStream_t st) {
  CmArgs a{};
  a.B = r.B;
  a.C = r.C;
  a.H = r.H;
  a.W = r.W;
  a.nWx = (r.W + CW - 1) / CW;
  a.nWin = a.nWx * ((r.H + CW - 1) / CW);
  a.wupc = (int)(((long long)r.B * a.nWin + 15) / 16);
  a.total = (long long)r.C * a.wupc;
  a.x = (const float*)r.x;
  a.M = (const float*)r.M;
  a.out = out;
  a.out2 = out2;
  const long long rounds = (a.total + kCmWaves - 1) / kCmWaves;
  const int cus = cm_cu_count();
  int grid = (int)(rounds < cus ? rounds : cus);
  // Few channels with many wave-units each: splitting every channel into `parts` workgroups
  // (one matrix staging each) beats contiguous ranges, whose workgroups straddle a channel
  // boundary (a second staging and a partial round), when it needs no more rounds per workgroup.
  a.parts = 0;
  if (r.C <= cus) {
    const int parts = (int)std::min<long long>(cus / r.C, a.wupc);
    const long long per = (a.wupc + parts - 1) / parts;
    const long long rounds_split = (per + kCmWaves - 1) / kCmWaves;
    const long long per_range = (a.total + grid - 1) / grid;
    const long long rounds_range = (per_range + kCmWaves - 1) / kCmWaves + 1;  // + a straddle
    if (rounds_split <= rounds_range && (long long)r.C * parts <= 0x7fffffffLL) {
      a.parts = parts;
      grid = r.C * parts;
    }
  }
  hipError_t e = hipFuncSetAttribute((const void*)k_fwd_cm,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, kCmLds);
  if (e != hipSuccess) return e;
  return launch_main(k_fwd_cm, dim3(grid), dim3(kCmThreads), kCmLds, st, a);
}

}  // namespace wbmm
