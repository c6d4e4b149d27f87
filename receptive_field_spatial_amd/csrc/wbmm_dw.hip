// Standard k x k depthwise convolution (DW-Std) on gfx950, fp32, NCHW: the gather-based operator
// the pages time WBMM against. Every output sums the k*k neighbours around its own position in
// its own channel [pith page, Fig. 1 and Fig. 2 captions; operator benchmark: Fig. 3 caption].
// y[b,c,h,v] = sum_{u,t} W[c,u,t] * x[b,c,h+u-p,v+t-p], p = k / 2, zeros outside the image.
//
// Work items are bands of RY-row tiles of one plane (b, c). Each item's input rows, with a zero
// halo of p pixels on every side, are staged once in LDS (the only HBM read of x); then every
// lane computes an RY x 4 output tile: for each kernel row u (its k weights wave-uniform, in
// scalar registers) and each of the tile's rows, one input row segment of k + 3 values comes from
// LDS as 16-byte reads and feeds 4k FMAs. Walking u outermost keeps only k weights live (all k*k
// of a 13 x 13 kernel would not fit the scalar registers). A workgroup holds up to four items,
// one or more waves each, so small planes still fill whole waves.
#include "wbmm_device.hpp"
#include "wbmm_launch.hpp"

namespace wbmm {

namespace {

constexpr int kDwRX = 4;  // output columns per lane

struct DwGeo {
  int B, C, H, W;
  int ry;         // output rows per lane (4 or 7)
  int tpr;        // tiles per row (ceil(W / 4))
  int br;         // tile rows per band
  int nbands;     // bands per plane
  int band_tiles; // br * tpr <= 64 * wpi
  int wpi;        // waves per item
  int ipw;        // items per workgroup
  int pw, ph;     // LDS pitch (floats, multiple of 4) and rows per item
  int vec4;       // W % 4 == 0 and 16-byte aligned x, y: staging and stores as 16-byte accesses
  long long items;
};

struct DwArgs {
  DwGeo g;
  const float* x;
  const float* w;
  float* y;
};

template <int K, int RY>
__global__ void __launch_bounds__(kThreads) k_dw_conv(DwArgs a) {
  extern __shared__ __attribute__((aligned(16))) float smem_f[];
  constexpr int P = K / 2, RX = kDwRX, NQ = (RX + K - 1 + 3) / 4;  // 16-byte reads per row
  const DwGeo& g = a.g;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int local = wave / g.wpi;  // item within the workgroup (wave-uniform; blockDim = ipw*wpi*64)
  const long long it = (long long)blockIdx.x * g.ipw + local;
  const bool live = it < g.items;
  const int plane = live ? (int)(it / g.nbands) : 0;
  const int band = live ? (int)(it % g.nbands) : 0;
  const int c = plane % g.C;
  const int pt = (wave % g.wpi) * 64 + lane;  // thread within the item
  const int nt = g.wpi * 64;                  // >= band_tiles
  const int h0 = band * g.br * RY;            // first output row of the band
  float* slab = smem_f + (size_t)local * g.ph * g.pw;
  const float* xp = a.x + (size_t)plane * g.H * g.W;

  // ---- stage LDS rows r = 0 .. ph-1 (image row h0 - P + r); LDS column P + v holds image
  //      column v, zero outside the image. Four columns per group; each lane takes groups in
  //      batches of SB with every load of a batch in flight before its LDS writes.
  constexpr int SB = 8;
  const int gpr = g.pw / 4, total = g.ph * gpr;
  for (int e0 = 0; e0 < total; e0 += SB * nt) {
    float v[SB][4];
    if (g.vec4) {  // group q: image columns 4q .. 4q+3 (one 16-byte load) -> LDS 4q+P ..
#pragma unroll
      for (int s = 0; s < SB; ++s) {
        const int e = e0 + s * nt + pt;
        const int r = e / gpr, q = e - r * gpr;
        const int hh = h0 - P + r, v0 = 4 * q;
        const bool in = live && e < total && hh >= 0 && hh < g.H && v0 < g.W;
        const v4f t4 = *(const v4f*)(xp + (in ? (size_t)hh * g.W + v0 : 0));
#pragma unroll
        for (int j = 0; j < 4; ++j) v[s][j] = in ? t4[j] : 0.f;
      }
#pragma unroll
      for (int s = 0; s < SB; ++s) {
        const int e = e0 + s * nt + pt;
        if (e >= total) break;
        const int r = e / gpr, q = e - r * gpr;
        float* dst = slab + r * g.pw + P + 4 * q;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (4 * q + P + j < g.pw) dst[j] = v[s][j];
        if (q == 0) {
#pragma unroll
          for (int j = 0; j < P; ++j) slab[r * g.pw + j] = 0.f;
        }
      }
    } else {  // group q: LDS columns 4q .. 4q+3, image columns 4q - P .., one load each
#pragma unroll
      for (int s = 0; s < SB; ++s) {
        const int e = e0 + s * nt + pt;
        const int r = e / gpr, q = e - r * gpr;
        const int hh = h0 - P + r;
        const bool row_in = live && e < total && hh >= 0 && hh < g.H;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int vv = 4 * q + j - P;
          const bool in = row_in && vv >= 0 && vv < g.W;
          const float t = xp[in ? (size_t)hh * g.W + vv : 0];
          v[s][j] = in ? t : 0.f;
        }
      }
#pragma unroll
      for (int s = 0; s < SB; ++s) {
        const int e = e0 + s * nt + pt;
        if (e >= total) break;
        const int r = e / gpr, q = e - r * gpr;
        *(v4f*)(slab + r * g.pw + 4 * q) = v4f{v[s][0], v[s][1], v[s][2], v[s][3]};
      }
    }
  }
  __syncthreads();
  const int t = pt;
  const int ty = t / g.tpr, tx = t - ty * g.tpr;
  const int oy0 = h0 + ty * RY, ox0 = tx * RX;
  if (!live || t >= g.band_tiles || oy0 >= g.H) return;

  // the channel's weights through the constant address space: wave-uniform, so scalar loads
  typedef const __attribute__((address_space(4))) float cfloat;
  cfloat* wc = (cfloat*)(a.w + (size_t)c * K * K);
  // LDS column of the first input the tile reads (image column ox0 - P): ox0, a multiple of 4
  const float* base = slab + (ty * RY) * g.pw + ox0;
  float acc[RY][RX];
#pragma unroll
  for (int i = 0; i < RY; ++i)
#pragma unroll
    for (int j = 0; j < RX; ++j) acc[i][j] = 0.f;
  // Kernel rows u run as a loop (its k weights: scalar loads, one row ahead); inside,
  // the tile's RY rows are unrolled and software-pipelined one row ahead: input row oy + u
  // (LDS columns ox0 .. ox0 + 4*NQ - 1, i.e. image columns ox0 - P ..) as NQ 16-byte reads.
  // The row offset passes through an empty asm and the accumulators are pinned after each row
  // step, so the reads and FMAs stay in their step and only two rows are live (left alone, the
  // compiler hoists every read of the unrolled rows and runs out of registers).
  float wn[K];  // weights of the next kernel row, loaded one row ahead
#pragma unroll
  for (int v = 0; v < K; ++v) wn[v] = wc[v];
#pragma unroll 1
  for (int u = 0; u < K; ++u) {
    float wu[K];
#pragma unroll
    for (int v = 0; v < K; ++v) wu[v] = wn[v];
    const int un = u + 1 < K ? u + 1 : u;  // the last row reloads itself (unused)
#pragma unroll
    for (int v = 0; v < K; ++v) wn[v] = wc[un * K + v];
    v4f rb[2][NQ];  // rows in flight and in use, alternating by row parity (no copies)
    auto load_row = [&](int r, v4f (&dst)[NQ]) {
      int off = r * g.pw;
      asm volatile("" : "+v"(off));
#pragma unroll
      for (int q = 0; q < NQ; ++q) dst[q] = *(const v4f*)(base + off + 4 * q);
    };
    load_row(u, rb[0]);
#pragma unroll
    for (int oy = 0; oy < RY; ++oy) {
      if (oy + 1 < RY) load_row(oy + 1 + u, rb[(oy + 1) & 1]);
      const v4f(&cur)[NQ] = rb[oy & 1];
#pragma unroll
      for (int v = 0; v < K; ++v)
#pragma unroll
        for (int ox = 0; ox < RX; ++ox)
          acc[oy][ox] = fmaf(wu[v], cur[(ox + v) / 4][(ox + v) % 4], acc[oy][ox]);
      asm volatile("" : "+v"(acc[oy][0]), "+v"(acc[oy][1]), "+v"(acc[oy][2]), "+v"(acc[oy][3]));
    }
  }
  // ---- store: a tile row is one 16-byte store when the row is whole and 16-byte aligned
  float* yp = a.y + (size_t)plane * g.H * g.W;
  const bool whole = g.vec4 && ox0 + RX <= g.W;
#pragma unroll
  for (int oy = 0; oy < RY; ++oy) {
    const int h = oy0 + oy;
    if (h >= g.H) break;
    float* o = yp + (size_t)h * g.W + ox0;
    if (whole) {
      *(v4f*)o = v4f{acc[oy][0], acc[oy][1], acc[oy][2], acc[oy][3]};
    } else {
#pragma unroll
      for (int ox = 0; ox < RX; ++ox)
        if (ox0 + ox < g.W) o[ox] = acc[oy][ox];
    }
  }
}

// Lanes used / lanes launched for RY-row tiles of a W-wide plane of H rows.
double dw_util(int H, int W, int ry) {
  const int tpr = (W + kDwRX - 1) / kDwRX, trows = (H + ry - 1) / ry;
  int br = 256 / tpr;
  if (br > trows) br = trows;
  const int tiles = br * tpr;
  return (double)tiles / (((tiles + 63) / 64) * 64);
}

bool plan_dw(DwGeo& g, int B, int C, int H, int W, int k, const void* x, const void* y) {
  const int p = k / 2, RX = kDwRX;
  g.B = B;
  g.C = C;
  g.H = H;
  g.W = W;
  g.ry = dw_util(H, W, 7) >= dw_util(H, W, 4) ? 7 : 4;
  g.tpr = (W + RX - 1) / RX;
  if (g.tpr > 256) return false;  // one tile per lane, at most 4 waves per item
  const int trows = (H + g.ry - 1) / g.ry;
  g.br = 256 / g.tpr;
  if (g.br > trows) g.br = trows;
  g.nbands = (trows + g.br - 1) / g.br;
  g.band_tiles = g.br * g.tpr;
  g.wpi = (g.band_tiles + 63) / 64;
  g.ipw = 4 / g.wpi;
  // the last tile reads LDS columns up to tpr*4 + 2p - 1
  g.pw = (g.tpr * RX + 2 * p + 3) / 4 * 4;
  g.ph = g.br * g.ry + k - 1;
  g.vec4 = (W % 4 == 0 && ((uintptr_t)x & 15) == 0 && ((uintptr_t)y & 15) == 0) ? 1 : 0;
  g.items = (long long)B * C * g.nbands;
  const size_t lds = (size_t)g.ipw * g.ph * g.pw * sizeof(float);
  return lds <= 64 * 1024 && (long long)B * C < (1LL << 31) &&
         (g.items + g.ipw - 1) / g.ipw < (1LL << 31);
}

template <int K, int RY>
hipError_t launch_dw_t(const DwArgs& a, hipStream_t st) {
  const unsigned lds = (unsigned)(a.g.ipw * a.g.ph * a.g.pw * sizeof(float));
  const unsigned grid = (unsigned)((a.g.items + a.g.ipw - 1) / a.g.ipw);
  return launch_main(k_dw_conv<K, RY>, dim3(grid), dim3(a.g.ipw * a.g.wpi * 64), lds, st, a);
}

template <int K>
hipError_t launch_dw_k(const DwArgs& a, hipStream_t st) {
  return a.g.ry == 7 ? launch_dw_t<K, 7>(a, st) : launch_dw_t<K, 4>(a, st);
}

}  // namespace

bool dwconv_supported(int B, int C, int H, int W, int k) {
  if (k < 3 || k > 13 || (k & 1) == 0) return false;
  DwGeo g;
  return plan_dw(g, B, C, H, W, k, nullptr, nullptr);
}

hipError_t launch_dwconv(int B, int C, int H, int W, int k, const float* x, const float* w,
                         float* y, hipStream_t st) {
  DwArgs a{};
  if (!plan_dw(a.g, B, C, H, W, k, x, y)) return hipErrorInvalidValue;
  a.x = x;
  a.w = w;
  a.y = y;
  switch (k) {
    case 3: return launch_dw_k<3>(a, st);
    case 5: return launch_dw_k<5>(a, st);
    case 7: return launch_dw_k<7>(a, st);
    case 9: return launch_dw_k<9>(a, st);
    case 11: return launch_dw_k<11>(a, st);
    case 13: return launch_dw_k<13>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace wbmm
