// Offset (interleaved) window grids on the fast kernels.
//
// WBMM acts on each window of a channel on its own, with that channel's table (WBMM paper, the
// windowed product and its matrix M built from the table T), so the windows of an offset grid
// (first window at (-oy, -ox), pixels outside the image zero) can be moved anywhere before the
// product and moved back after it. This path copies the grid's windows of every channel into
// whole 28 x 28 images of 2 x 2 windows (w = 14) in the workspace, runs the fast kernels there
// without the mix (fp32 maps; bf16 maps without the mix go to the fast bf16 forward), and
// copies the result back to image coordinates, where the 3 x 3 mix runs
// on the whole map as its own pass. The backward does the same with the mix's data gradient G
// and X; the table gradient is a sum over windows, whose zero pixels add nothing.
//
// Global window n = b * nW + wy * nwx + wx of image b sits in repacked image q = n / 4 at
// window slot n % 4 (row-major 2 x 2); windows past B * nW are zero.
#include "wbmm_device.hpp"
#include "wbmm_launch.hpp"

namespace wbmm {
namespace {

constexpr int kW = 14;          // window side of this path
constexpr int kP = 2 * kW;      // repacked image side
constexpr int kQ = kP * kP / 4; // float4 per repacked plane

struct RepackGeo {
  int B, C, H, W, oy, ox, nwx, nW, Bp;
};

RepackGeo repack_geo(int B, int C, int H, int W, int oy, int ox) {
  RepackGeo g{};
  g.B = B;
  g.C = C;
  g.H = H;
  g.W = W;
  g.oy = oy;
  g.ox = ox;
  g.nwx = (W + ox + kW - 1) / kW;
  g.nW = ((H + oy + kW - 1) / kW) * g.nwx;
  g.Bp = (int)(((long long)B * g.nW + 3) / 4);
  return g;
}

bool repack_fits(int B, int C, int H, int W, int w, int layout, int oy, int ox) {
  if (w != kW || layout != 0 || (oy == 0 && ox == 0) || B < 1 || C < 1 || H < 1 || W < 1)
    return false;
  const long long nW = (long long)((H + oy + kW - 1) / kW) * ((W + ox + kW - 1) / kW);
  const long long Bp = ((long long)B * nW + 3) / 4;
  return Bp * C * kQ < (1LL << 31) && (long long)C * H * W < (1LL << 31) &&
         (long long)B * C < (1LL << 31) && offsets_fit(C, kP, kP);
}

size_t al256(size_t v) { return (v + 255) / 256 * 256; }
size_t repacked_bytes(const RepackGeo& g, size_t esz = 4) {
  return al256((size_t)g.Bp * g.C * kP * kP * esz);
}

// four map elements as one store: float4 (fp32) or 4 x 16 bits (bf16)
__device__ __forceinline__ void put4(float* p, const float (&v)[4]) {
  *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void put4(uint16_t* p, const uint16_t (&v)[4]) {
  *(uint2*)p = make_uint2(v[0] | ((uint32_t)v[1] << 16), v[2] | ((uint32_t)v[3] << 16));
}
bool mix_planes_fit(int H, int W) { return mix_bwd_pass_ok(H, W); }
size_t mix_partials_bytes(int B, int C, int H, int W) {
  return al256((size_t)C * mix_bwd_parts(B, H, W) * 9 * sizeof(double));
}

// Repacked map <- image map: workgroup (qg, c) takes repacked planes (q, c) for
// q = kGQ qg .. kGQ qg + kGQ - 1 (consecutive windows of a channel: their source rows share cache
// lines). Each plane's 4 windows are located once (uniform); each thread then loads one float4
// of a repacked row (4 pixels, which may lie in two windows) of every plane, all loads in flight
// before the stores. Pixels outside the image or past the last window are 0.
constexpr int kGQ = 4;

template <typename TE>
__global__ void __launch_bounds__(256) k_gather_windows(RepackGeo g, const TE* __restrict__ src,
                                                        TE* __restrict__ dst) {
  const int qg = blockIdx.x / g.C, c = blockIdx.x - qg * g.C;
  const int nlast = g.B * g.nW;  // 4 Bp < 2^31: window numbers fit in 32 bits
  const int j = threadIdx.x;
  const int py = j / (kP / 4), px0 = (j - py * (kP / 4)) * 4;
  const int ky = py / kW, y = py - ky * kW;
  TE v[kGQ][4];
#pragma unroll
  for (int i = 0; i < kGQ; ++i) {
    const int q = kGQ * qg + i;
    // the row's two window slots 2 ky (left) and 2 ky + 1 (right): source plane offset (-1: past
    // the last window) and the image position of the window's first pixel
    long long sb[2];
    int oy2[2], ox2[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int n = 4 * q + 2 * ky + h;
      const int b = n / g.nW, kk = n - b * g.nW;
      const int wy = kk / g.nwx, wx = kk - wy * g.nwx;
      sb[h] = (q < g.Bp && n < nlast) ? ((long long)b * g.C + c) * g.H * g.W : -1;
      oy2[h] = wy * kW - g.oy + y;
      ox2[h] = wx * kW - g.ox;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int px = px0 + e;
      const int h = px >= kW ? 1 : 0;
      const long long base = h ? sb[1] : sb[0];
      const int iy = h ? oy2[1] : oy2[0], ix = (h ? ox2[1] : ox2[0]) + px - h * kW;
      v[i][e] = TE(0);  // +0 in both types
      if (j < kQ && base >= 0 && iy >= 0 && iy < g.H && ix >= 0 && ix < g.W)
        v[i][e] = src[(size_t)base + (size_t)iy * g.W + ix];
    }
  }
  if (j >= kQ) return;
#pragma unroll
  for (int i = 0; i < kGQ; ++i) {
    const int q = kGQ * qg + i;
    if (q < g.Bp) put4(dst + (((size_t)q * g.C + c) * kQ + j) * 4, v[i]);
  }
}

// Image map <- repacked map: every image pixel lies in exactly one window of the grid. Workgroup
// (bg, c) takes the planes (b, c) for b = kSB bg .. kSB bg + kSB - 1, a row by 32 lanes (W <= 32)
// or by a wave, a pixel's kSB planes loaded before they are stored. dst2 (may be null) receives
// a second copy.
constexpr int kSB = 4;

template <typename TE>
__global__ void __launch_bounds__(256) k_scatter_windows(RepackGeo g, const TE* __restrict__ src,
                                                         TE* __restrict__ dst,
                                                         TE* __restrict__ dst2) {
  const int bg = blockIdx.x / g.C, c = blockIdx.x - bg * g.C;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool half = g.W <= 32;
  const int rows_per_pass = half ? 8 : 4, step = half ? 32 : 64;
  const int r0 = half ? 2 * wave + (lane >> 5) : wave, l0 = half ? (lane & 31) : lane;
  for (int iy = r0; iy < g.H; iy += rows_per_pass) {
    const int wy = (iy + g.oy) / kW, y = iy + g.oy - wy * kW;
    for (int ix = l0; ix < g.W; ix += step) {
      const int wx = (ix + g.ox) / kW, x = ix + g.ox - wx * kW;
      TE v[kSB];
#pragma unroll
      for (int i = 0; i < kSB; ++i) {
        const int b = kSB * bg + i;
        const int n = b * g.nW + wy * g.nwx + wx;
        const int q = n >> 2, k = n & 3;
        v[i] = b < g.B ? src[((size_t)q * g.C + c) * (kP * kP) + ((k >> 1) * kW + y) * kP +
                             (k & 1) * kW + x]
                       : TE(0);
      }
#pragma unroll
      for (int i = 0; i < kSB; ++i) {
        const int b = kSB * bg + i;
        if (b >= g.B) break;
        const size_t o = (((size_t)b * g.C + c) * g.H + iy) * g.W + ix;
        dst[o] = v[i];
        if (dst2) dst2[o] = v[i];
      }
    }
  }
}

template <typename TE>
hipError_t gather(const RepackGeo& g, const TE* src, TE* dst, hipStream_t st) {
  static_assert(kQ <= 256, "a repacked row's float4s per thread");
  const int groups = (g.Bp + kGQ - 1) / kGQ;
  hipLaunchKernelGGL(k_gather_windows<TE>, dim3(groups * g.C), dim3(256), 0, st, g, src, dst);
  return hipGetLastError();
}

template <typename TE>
hipError_t scatter(const RepackGeo& g, const TE* src, TE* dst, TE* dst2, hipStream_t st) {
  const int groups = (g.B + kSB - 1) / kSB;
  hipLaunchKernelGGL(k_scatter_windows<TE>, dim3(groups * g.C), dim3(256), 0, st, g, src, dst,
                     dst2);
  return hipGetLastError();
}

}  // namespace

bool repack_forward_ok(const FwdRequest& r) {
  const bool f32 = !r.in_bf16 && !r.out_bf16, bf16 = r.in_bf16 && r.out_bf16 && !r.mixw;
  return (f32 || bf16) && r.T && !r.M && !r.Tsub &&
         repack_fits(r.B, r.C, r.H, r.W, r.w, r.layout, r.oy, r.ox);
}

// [repacked X] [repacked z] [image-space z: with the mix and no fp32 z_save]
size_t repack_forward_workspace(const FwdRequest& r) {
  if (!repack_forward_ok(r)) return 0;
  const RepackGeo g = repack_geo(r.B, r.C, r.H, r.W, r.oy, r.ox);
  const bool zb = r.mixw && !r.zsave;
  return 2 * repacked_bytes(g, r.in_bf16 ? 2 : 4) +
         (zb ? al256((size_t)r.B * r.C * r.H * r.W * 4) : 0);
}

hipError_t launch_forward_repacked(const FwdRequest& r, hipStream_t st) {
  if (!repack_forward_ok(r)) return hipErrorInvalidValue;
  const RepackGeo g = repack_geo(r.B, r.C, r.H, r.W, r.oy, r.ox);
  unsigned char* ws = (unsigned char*)r.ws;
  FwdRequest q = r;
  q.B = g.Bp;
  q.H = q.W = kP;
  q.oy = q.ox = 0;
  q.zsave = nullptr;
  if (r.in_bf16) {  // bf16 maps, no mix: the fast bf16 forward on the repacked images
    uint16_t* xr = (uint16_t*)ws;
    uint16_t* zr = (uint16_t*)(ws + repacked_bytes(g, 2));
    q.x = xr;
    q.y = zr;
    if (!fast_bf16_forward_ok(q)) return hipErrorInvalidValue;
    hipError_t e = gather(g, (const uint16_t*)r.x, xr, st);
    if (e != hipSuccess) return e;
    e = launch_forward_fast_bf16(q, st);
    if (e != hipSuccess) return e;
    return scatter(g, (const uint16_t*)zr, (uint16_t*)r.y, (uint16_t*)r.zsave, st);
  }
  float* xr = (float*)ws;
  float* zr = (float*)(ws + repacked_bytes(g));
  hipError_t e = gather(g, (const float*)r.x, xr, st);
  if (e != hipSuccess) return e;
  q.x = xr;
  q.mixw = nullptr;
  q.y = zr;
  if (!fast_forward_ok(q)) return hipErrorInvalidValue;
  e = launch_forward_fast(q, st);
  if (e != hipSuccess) return e;
  if (!r.mixw) return scatter(g, (const float*)zr, (float*)r.y, (float*)r.zsave, st);
  float* z = r.zsave ? (float*)r.zsave : (float*)(ws + 2 * repacked_bytes(g));
  e = scatter(g, (const float*)zr, z, (float*)nullptr, st);
  if (e != hipSuccess) return e;
  if (mix_planes_fit(r.H, r.W))
    return launch_mix_fwd_planes_f32(z, r.mixw, (float*)r.y, r.B, r.C, r.H, r.W, st);
  return launch_mix_fwd(z, r.mixw, r.y, 0, r.B, r.C, r.H, r.W, 0, st);
}

namespace {
// With the mix: its data gradient G (and its weight gradient) on the whole map, in `ws` (the
// G map, then the dWmix partials); returns the map the product's backward reads (G, or dy).
hipError_t mix_adjoint_map(const BwdRequest& r, unsigned char* ws, const float** gsrc,
                           hipStream_t st) {
  *gsrc = r.dy;
  if (!r.mixw) return hipSuccess;
  float* gz = (float*)ws;
  hipError_t e;
  if (mix_planes_fit(r.H, r.W)) {  // one plane-staged pass: G and per-group dWmix partials
    double* partW = (double*)(ws + al256((size_t)r.B * r.C * r.H * r.W * 4));
    e = launch_mix_bwd_planes_f32(r.dy, r.dmixw ? r.zsaved : nullptr, r.mixw, gz, partW, r.B,
                                  r.C, r.H, r.W, st);
    if (e != hipSuccess) return e;
    if (r.dmixw) {
      e = launch_bwd_reduce(nullptr, partW, mix_bwd_parts(r.B, r.H, r.W), r.C, 0, nullptr,
                            r.dmixw, st);
      if (e != hipSuccess) return e;
    }
  } else {
    e = launch_mix_bwd_data(r.dy, r.mixw, gz, r.B, r.C, r.H, r.W, 0, st);
    if (e != hipSuccess) return e;
    if (r.dmixw) {
      e = launch_mix_bwd_weight(r.dy, r.zsaved, r.dmixw, r.B, r.C, r.H, r.W, 0, st);
      if (e != hipSuccess) return e;
    }
  }
  *gsrc = gz;
  return hipSuccess;
}
size_t mix_adjoint_bytes(const BwdRequest& r) {
  return r.mixw ? al256((size_t)r.B * r.C * r.H * r.W * 4) + mix_partials_bytes(r.B, r.C, r.H, r.W)
                : 0;
}
}  // namespace

bool repack_backward_ok(const BwdRequest& r) {
  return r.T && !r.M && !r.Tsub && repack_fits(r.B, r.C, r.H, r.W, r.w, r.layout, r.oy, r.ox);
}

namespace {
BwdRequest repacked_request(const BwdRequest& r, const RepackGeo& g) {
  BwdRequest q = r;
  q.B = g.Bp;
  q.H = q.W = kP;
  q.oy = q.ox = 0;
  q.mixw = nullptr;
  q.zsaved = nullptr;
  q.dmixw = nullptr;
  return q;
}
}  // namespace

// [fast backward partials] [repacked G] [repacked X] [repacked dX]
// [with the mix: image-space G, dWmix partials of the plane-staged pass]
size_t repack_backward_workspace(const BwdRequest& r) {
  if (!repack_backward_ok(r)) return 0;
  const RepackGeo g = repack_geo(r.B, r.C, r.H, r.W, r.oy, r.ox);
  const size_t fast = al256(fast_backward_workspace(repacked_request(r, g)));
  return fast + 3 * repacked_bytes(g) + mix_adjoint_bytes(r);
}

// The rolled-map kernels for grid offsets 0 or 7 on 28 x 28 maps (fp32):
// [table-gradient partials] [with the mix: G map, dWmix partials]
bool roll_backward_ok(const BwdRequest& r) { return fast_roll_backward_ok(r); }

size_t roll_backward_workspace(const BwdRequest& r) {
  if (!roll_backward_ok(r)) return 0;
  return al256(fast_roll_backward_workspace(r)) + mix_adjoint_bytes(r);
}

hipError_t launch_backward_rolled(const BwdRequest& r, hipStream_t st) {
  if (!roll_backward_ok(r)) return hipErrorInvalidValue;
  unsigned char* ws = (unsigned char*)r.ws;
  const size_t part = al256(fast_roll_backward_workspace(r));
  const float* gsrc = nullptr;
  hipError_t e = mix_adjoint_map(r, ws + part, &gsrc, st);
  if (e != hipSuccess || (!r.dx && !r.dT)) return e;
  BwdRequest q = r;
  q.dy = gsrc;
  q.mixw = nullptr;
  q.zsaved = nullptr;
  q.dmixw = nullptr;
  q.ws = ws;
  return launch_backward_fast_roll(q, st);
}

hipError_t launch_backward_repacked(const BwdRequest& r, hipStream_t st) {
  if (!repack_backward_ok(r)) return hipErrorInvalidValue;
  const RepackGeo g = repack_geo(r.B, r.C, r.H, r.W, r.oy, r.ox);
  BwdRequest q = repacked_request(r, g);
  if (!fast_backward_ok(q)) return hipErrorInvalidValue;
  unsigned char* ws = (unsigned char*)r.ws;
  const size_t fast = al256(fast_backward_workspace(q));
  const size_t rb = repacked_bytes(g);
  float* gr = (float*)(ws + fast);
  float* xr = (float*)(ws + fast + rb);
  float* dxr = (float*)(ws + fast + 2 * rb);
  const float* gsrc = nullptr;
  hipError_t e = mix_adjoint_map(r, ws + fast + 3 * rb, &gsrc, st);
  if (e != hipSuccess) return e;
  if (!r.dx && !r.dT) return hipSuccess;
  e = gather<float>(g, gsrc, gr, st);
  if (e != hipSuccess) return e;
  e = gather<float>(g, r.x, xr, st);
  if (e != hipSuccess) return e;
  q.x = xr;
  q.dy = gr;
  q.dx = r.dx ? dxr : nullptr;
  q.ws = ws;
  e = launch_backward_fast(q, st);
  if (e != hipSuccess || !r.dx) return e;
  return scatter(g, (const float*)dxr, r.dx, (float*)nullptr, st);
}

}  // namespace wbmm
