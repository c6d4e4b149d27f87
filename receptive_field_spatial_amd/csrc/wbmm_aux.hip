// Index/matrix construction, hierarchical fold and the stand-alone 3x3 mix passes.
#include "wbmm_device.hpp"
#include "wbmm_launch.hpp"
#include "wbmm_plan.hpp"

namespace wbmm {

namespace {

inline unsigned grid_for(size_t n, unsigned per_block = kThreads, unsigned cap = 65536u) {
  size_t b = (n + per_block - 1) / per_block;
  if (b < 1) b = 1;
  return (unsigned)(b > cap ? cap : b);
}

}  // namespace

// idx[i*d + j] = (y_i - y_j + w - 1)(2w - 1) + (x_i - x_j + w - 1)
// [gecl.asia reading notes, "Core Idea": a relative-position table indexed by the in-window offset]
__global__ void __launch_bounds__(kThreads) k_build_index(int w, int32_t* idx) {
  const int d = w * w, L1 = 2 * w - 1;
  const int total = d * d;
  for (int e = blockIdx.x * kThreads + threadIdx.x; e < total; e += gridDim.x * kThreads) {
    const int i = e / d, j = e - (e / d) * d;
    const int yi = i / w, xi = i - (i / w) * w, yj = j / w, xj = j - (j / w) * w;
    idx[e] = (yi - yj + w - 1) * L1 + (xi - xj + w - 1);
  }
}

// M[c][i][j] = T[c][idx(i, j)]: an exact element copy (E = float or bf16 bits).
template <typename E>
__global__ void __launch_bounds__(kThreads) k_build_matrix(const E* __restrict__ T, int C, int w,
                                                           FastDiv fd_d, FastDiv fd_w,
                                                           E* __restrict__ M) {
  const int d = w * w, L1 = 2 * w - 1, L = L1 * L1;
  const size_t dd = (size_t)d * d;
  const size_t total = (size_t)C * dd;
  for (size_t e = (size_t)blockIdx.x * kThreads + threadIdx.x; e < total;
       e += (size_t)gridDim.x * kThreads) {
    const size_t c = e / dd;
    const uint32_t ij = (uint32_t)(e - c * dd);
    uint32_t i, j, yi, xi, yj, xj;
    fdivmod(ij, fd_d, i, j);
    fdivmod(i, fd_w, yi, xi);
    fdivmod(j, fd_w, yj, xj);
    const int q = ((int)yi - (int)yj + w - 1) * L1 + ((int)xi - (int)xj + w - 1);
    M[e] = T[c * L + q];
  }
}

// Hierarchical fold: same-sub-window pairs get one added table entry (fp32 add, RNE; for bf16 the
// two bf16 values are added in fp32 and the sum is rounded to bf16)
// [gecl.asia reading notes, "Method" point 4].
// Min may be Mout (each element is read, then written, by one thread).
template <typename E>
__global__ void __launch_bounds__(kThreads) k_fold(const E* Min,
                                                   const E* __restrict__ Ts, int C, int w, int s,
                                                   FastDiv fd_d, FastDiv fd_w, FastDiv fd_s,
                                                   E* Mout) {
  const int d = w * w, Ls1 = 2 * s - 1, Ls = Ls1 * Ls1;
  const size_t dd = (size_t)d * d;
  const size_t total = (size_t)C * dd;
  for (size_t e = (size_t)blockIdx.x * kThreads + threadIdx.x; e < total;
       e += (size_t)gridDim.x * kThreads) {
    const size_t c = e / dd;
    const uint32_t ij = (uint32_t)(e - c * dd);
    uint32_t i, j, yi, xi, yj, xj, byi, ryi, bxi, rxi, byj, ryj, bxj, rxj;
    fdivmod(ij, fd_d, i, j);
    fdivmod(i, fd_w, yi, xi);
    fdivmod(j, fd_w, yj, xj);
    fdivmod(yi, fd_s, byi, ryi);
    fdivmod(xi, fd_s, bxi, rxi);
    fdivmod(yj, fd_s, byj, ryj);
    fdivmod(xj, fd_s, bxj, rxj);
    E m = Min[e];
    if (byi == byj && bxi == bxj) {
      const int q = ((int)ryi - (int)ryj + s - 1) * Ls1 + ((int)rxi - (int)rxj + s - 1);
      if constexpr (sizeof(E) == 4) {
        m = m + Ts[c * Ls + q];
      } else {
        m = f2bf(bf2f(m) + bf2f(Ts[c * Ls + q]));
      }
    }
    Mout[e] = m;
  }
}

hipError_t launch_build_index(int w, int32_t* idx, hipStream_t st) {
  const size_t n = (size_t)w * w * w * w;
  hipLaunchKernelGGL(k_build_index, dim3(grid_for(n)), dim3(kThreads), 0, st, w, idx);
  return hipGetLastError();
}

hipError_t launch_build_matrix(const void* T, int C, int w, int bf16, void* M, hipStream_t st) {
  const size_t n = (size_t)C * w * w * w * w;
  const FastDiv fd_d = make_fastdiv(w * w), fd_w = make_fastdiv(w);
  if (bf16)
    hipLaunchKernelGGL(k_build_matrix<uint16_t>, dim3(grid_for(n)), dim3(kThreads), 0, st,
                       (const uint16_t*)T, C, w, fd_d, fd_w, (uint16_t*)M);
  else
    hipLaunchKernelGGL(k_build_matrix<float>, dim3(grid_for(n)), dim3(kThreads), 0, st,
                       (const float*)T, C, w, fd_d, fd_w, (float*)M);
  return hipGetLastError();
}

hipError_t launch_fold(const void* Min, const void* Tsub, int C, int w, int s, int bf16,
                       void* Mout, hipStream_t st) {
  const size_t n = (size_t)C * w * w * w * w;
  const FastDiv fd_d = make_fastdiv(w * w), fd_w = make_fastdiv(w), fd_s = make_fastdiv(s);
  if (bf16)
    hipLaunchKernelGGL(k_fold<uint16_t>, dim3(grid_for(n)), dim3(kThreads), 0, st,
                       (const uint16_t*)Min, (const uint16_t*)Tsub, C, w, s, fd_d, fd_w, fd_s,
                       (uint16_t*)Mout);
  else
    hipLaunchKernelGGL(k_fold<float>, dim3(grid_for(n)), dim3(kThreads), 0, st,
                       (const float*)Min, (const float*)Tsub, C, w, s, fd_d, fd_w, fd_s,
                       (float*)Mout);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------- 3x3 mix passes
// Decompose a flat index of a (B, C, H, W) map in `layout` into (b, c, h, v).
__device__ __forceinline__ void map_coords(size_t e, int layout, int C, int H, int W, int& b,
                                           int& c, int& h, int& v) {
  if (layout == 0) {
    v = (int)(e % W); e /= W;
    h = (int)(e % H); e /= H;
    c = (int)(e % C); b = (int)(e / C);
  } else {
    c = (int)(e % C); e /= C;
    v = (int)(e % W); e /= W;
    h = (int)(e % H); b = (int)(e / H);
  }
}

// y[b,c,h,v] = sum_{u,t} w9[c][u][t] * z[b,c,h+u-1,v+t-1]  (zero outside the map)
// [gecl.asia reading notes, "Method" point 3: cross-block 3x3 depthwise mixing]
// zcopy (bf16, or null): the pre-mix map z rounded to bf16, for a bf16 z_save.
__global__ void __launch_bounds__(kThreads) k_mix_fwd(const float* __restrict__ z,
                                                      const float* __restrict__ w9, void* y,
                                                      int out_bf16, int B, int C, int H, int W,
                                                      int layout, uint16_t* zcopy) {
  const size_t total = (size_t)B * C * H * W;
  for (size_t e = (size_t)blockIdx.x * kThreads + threadIdx.x; e < total;
       e += (size_t)gridDim.x * kThreads) {
    int b, c, h, v;
    map_coords(e, layout, C, H, W, b, c, h, v);
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int hh = h + u - 1;
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const int vv = v + t - 1;
        const float zv = (hh >= 0 && hh < H && vv >= 0 && vv < W)
                             ? z[map_off(layout, b, c, hh, vv, C, H, W)] : 0.f;
        acc = fmaf(w9[c * 9 + u * 3 + t], zv, acc);
      }
    }
    if (out_bf16) ((uint16_t*)y)[e] = f2bf(acc);
    else ((float*)y)[e] = acc;
    if (zcopy) zcopy[e] = f2bf(z[e]);
  }
}

// dz[b,c,p,q] = sum_{u,t} w9[c][u][t] * dy[b,c,p-u+1,q-t+1]  (adjoint of k_mix_fwd); bf16
// maps (TM = uint16_t) are read and written as bf16 (RNE), the sums run in fp32.
template <typename TM>
__global__ void __launch_bounds__(kThreads) k_mix_bwd_data(const TM* __restrict__ dy,
                                                           const float* __restrict__ w9,
                                                           TM* __restrict__ dz, int B, int C,
                                                           int H, int W, int layout) {
  const size_t total = (size_t)B * C * H * W;
  for (size_t e = (size_t)blockIdx.x * kThreads + threadIdx.x; e < total;
       e += (size_t)gridDim.x * kThreads) {
    int b, c, h, v;
    map_coords(e, layout, C, H, W, b, c, h, v);
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int hh = h - u + 1;
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const int vv = v - t + 1;
        const float g = (hh >= 0 && hh < H && vv >= 0 && vv < W)
                            ? load_f32<TM>(dy, map_off(layout, b, c, hh, vv, C, H, W)) : 0.f;
        acc = fmaf(w9[c * 9 + u * 3 + t], g, acc);
      }
    }
    if constexpr (sizeof(TM) == 2) dz[e] = f2bf(acc);
    else dz[e] = acc;
  }
}

// dw9[c][u][t] = sum_{b,h,v} dy[b,c,h,v] * z[b,c,h+u-1,v+t-1]; one workgroup per channel,
// fp64 partial sums per thread, then a fixed-order tree: bitwise reproducible.
template <typename TM>
__global__ void __launch_bounds__(kThreads) k_mix_bwd_weight(const TM* __restrict__ dy,
                                                             const TM* __restrict__ z,
                                                             float* __restrict__ dw9, int B,
                                                             int C, int H, int W, int layout) {
  __shared__ double red[9][kThreads];
  const int c = blockIdx.x;
  double acc[9];
#pragma unroll
  for (int q = 0; q < 9; ++q) acc[q] = 0.0;
  const size_t per = (size_t)B * H * W;
  for (size_t e = threadIdx.x; e < per; e += kThreads) {
    const int v = (int)(e % W);
    const int h = (int)((e / W) % H);
    const int b = (int)(e / ((size_t)W * H));
    const double g = load_f32<TM>(dy, map_off(layout, b, c, h, v, C, H, W));
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int hh = h + u - 1;
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const int vv = v + t - 1;
        if (hh >= 0 && hh < H && vv >= 0 && vv < W)
          acc[u * 3 + t] += g * (double)load_f32<TM>(z, map_off(layout, b, c, hh, vv, C, H, W));
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 9; ++q) red[q][threadIdx.x] = acc[q];
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) {
#pragma unroll
      for (int q = 0; q < 9; ++q) red[q][threadIdx.x] += red[q][threadIdx.x + s];
    }
    __syncthreads();
  }
  if (threadIdx.x < 9) dw9[c * 9 + threadIdx.x] = (float)red[threadIdx.x][0];
}

// dT[c][q] = sum over partials k (in order) of partT[c][k][q]; the same for the 9 dWmix values
// over their own partials. Workgroup (c, j) takes entries q = 256 j .. 256 j + 255 of channel c
// (one per thread, so each thread waits for one batch of loads); workgroups with j = 0 also sum
// dWmix.
__global__ void __launch_bounds__(kThreads) k_bwd_reduce(const double* __restrict__ partT,
                                                         int partsT,
                                                         const double* __restrict__ partW,
                                                         int partsW, int L, float* __restrict__ dT,
                                                         float* __restrict__ dmixw) {
  const int c = blockIdx.x;
  // partials are loaded 8 at a time (all in flight together) and added in order k = 0, 1, ...
  auto sum = [](const double* p, size_t stride, int parts) {
    double s = 0.0;
    for (int k0 = 0; k0 < parts; k0 += 8) {
      double v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = k0 + j < parts ? p[(size_t)(k0 + j) * stride] : 0.0;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (k0 + j < parts) s += v[j];
    }
    return s;
  };
  const int q = blockIdx.y * kThreads + threadIdx.x;
  if (dT && q < L)
    dT[(size_t)c * L + q] = (float)sum(partT + (size_t)c * partsT * L + q, (size_t)L, partsT);
  if (dmixw && blockIdx.y == 0 && threadIdx.x < 9)
    dmixw[c * 9 + threadIdx.x] =
        (float)sum(partW + (size_t)c * partsW * 9 + threadIdx.x, 9, partsW);
}

hipError_t launch_bwd_reduce2(const double* partT, int partsT, const double* partW, int partsW,
                              int C, int L, float* dT, float* dmixw, hipStream_t st) {
  const int gy = dT && L > 0 ? (L + kThreads - 1) / kThreads : 1;
  hipLaunchKernelGGL(k_bwd_reduce, dim3(C, gy), dim3(kThreads), 0, st, partT, partsT, partW,
                     partsW, L, dT, dmixw);
  return hipGetLastError();
}

hipError_t launch_bwd_reduce(const double* partT, const double* partW, int parts, int C, int L,
                             float* dT, float* dmixw, hipStream_t st) {
  return launch_bwd_reduce2(partT, parts, partW, parts, C, L, dT, dmixw, st);
}

hipError_t launch_mix_fwd(const float* z, const float* w9, void* y, int out_bf16, int B, int C,
                          int H, int W, int layout, hipStream_t st, uint16_t* zcopy) {
  const size_t n = (size_t)B * C * H * W;
  hipLaunchKernelGGL(k_mix_fwd, dim3(grid_for(n)), dim3(kThreads), 0, st, z, w9, y, out_bf16, B,
                     C, H, W, layout, zcopy);
  return hipGetLastError();
}

hipError_t launch_mix_bwd_data(const float* dy, const float* w9, float* dz, int B, int C, int H,
                               int W, int layout, hipStream_t st) {
  const size_t n = (size_t)B * C * H * W;
  hipLaunchKernelGGL(k_mix_bwd_data<float>, dim3(grid_for(n)), dim3(kThreads), 0, st, dy, w9, dz,
                     B, C, H, W, layout);
  return hipGetLastError();
}

hipError_t launch_mix_bwd_weight(const float* dy, const float* z, float* dw9, int B, int C, int H,
                                 int W, int layout, hipStream_t st) {
  hipLaunchKernelGGL(k_mix_bwd_weight<float>, dim3(C), dim3(kThreads), 0, st, dy, z, dw9, B, C, H,
                     W, layout);
  return hipGetLastError();
}

template <typename TM>
hipError_t launch_mix_bwd_data_t(const TM* dy, const float* w9, TM* dz, int B, int C, int H,
                                 int W, int layout, hipStream_t st) {
  const size_t n = (size_t)B * C * H * W;
  hipLaunchKernelGGL(k_mix_bwd_data<TM>, dim3(grid_for(n)), dim3(kThreads), 0, st, dy, w9, dz, B,
                     C, H, W, layout);
  return hipGetLastError();
}

template <typename TM>
hipError_t launch_mix_bwd_weight_t(const TM* dy, const TM* z, float* dw9, int B, int C, int H,
                                   int W, int layout, hipStream_t st) {
  hipLaunchKernelGGL(k_mix_bwd_weight<TM>, dim3(C), dim3(kThreads), 0, st, dy, z, dw9, B, C, H, W,
                     layout);
  return hipGetLastError();
}

template hipError_t launch_mix_bwd_data_t<float>(const float*, const float*, float*, int, int, int,
                                                 int, int, hipStream_t);
template hipError_t launch_mix_bwd_data_t<uint16_t>(const uint16_t*, const float*, uint16_t*, int,
                                                    int, int, int, int, hipStream_t);
template hipError_t launch_mix_bwd_weight_t<float>(const float*, const float*, float*, int, int,
                                                   int, int, int, hipStream_t);
template hipError_t launch_mix_bwd_weight_t<uint16_t>(const uint16_t*, const uint16_t*, float*,
                                                      int, int, int, int, int, hipStream_t);

// Stage one plane (bf16 or fp32) into LDS as fp32 with a one-pixel zero halo (pitch W + 2): the
// halo is zeroed, then the interior is filled from pixel pairs (W even) or single pixels.
template <typename TM>
__device__ __forceinline__ void stage_plane(const TM* __restrict__ src, float* P, int H, int W);

template <>
__device__ __forceinline__ void stage_plane<uint16_t>(const uint16_t* __restrict__ src, float* P,
                                                      int H, int W) {
  const int PW = W + 2;
  for (int e = threadIdx.x; e < PW; e += kThreads) {
    P[e] = 0.f;
    P[(H + 1) * PW + e] = 0.f;
  }
  for (int r = threadIdx.x; r < H; r += kThreads) {
    P[(r + 1) * PW] = 0.f;
    P[(r + 1) * PW + W + 1] = 0.f;
  }
  if ((W & 1) == 0) {
    const int hw = W / 2;
    for (int e = threadIdx.x; e < H * hw; e += kThreads) {
      const int h = e / hw, v2 = e - h * hw;
      const uint32_t pr = *(const uint32_t*)(src + (size_t)h * W + 2 * v2);
      P[(h + 1) * PW + 2 * v2 + 1] = __uint_as_float(pr << 16);
      P[(h + 1) * PW + 2 * v2 + 2] = __uint_as_float(pr & 0xffff0000u);
    }
  } else {
    for (int e = threadIdx.x; e < H * W; e += kThreads) {
      const int h = e / W, v = e - h * W;
      P[(h + 1) * PW + v + 1] = bf2f(src[(size_t)h * W + v]);
    }
  }
}

template <>
__device__ __forceinline__ void stage_plane<float>(const float* __restrict__ src, float* P, int H,
                                                   int W) {
  const int PW = W + 2;
  for (int e = threadIdx.x; e < PW; e += kThreads) {
    P[e] = 0.f;
    P[(H + 1) * PW + e] = 0.f;
  }
  for (int r = threadIdx.x; r < H; r += kThreads) {
    P[(r + 1) * PW] = 0.f;
    P[(r + 1) * PW + W + 1] = 0.f;
  }
  if ((W & 1) == 0) {  // planes start at even pixel offsets: 8-byte pairs
    // large planes: eight pairs per thread in flight before their LDS writes (they would
    // otherwise pay one memory latency per pass); the loads are clamped, not guarded
    const int hw = W / 2, n = H * hw;
    if (n <= 4 * kThreads) {  // small planes: one or a few pairs per thread
      for (int e = threadIdx.x; e < n; e += kThreads) {
        const int h = e / hw, v2 = e - h * hw;
        const float2 pr = *(const float2*)(src + (size_t)h * W + 2 * v2);
        P[(h + 1) * PW + 2 * v2 + 1] = pr.x;
        P[(h + 1) * PW + 2 * v2 + 2] = pr.y;
      }
      return;
    }
    constexpr int KB = 8;
    for (int e0 = threadIdx.x; e0 < n; e0 += KB * kThreads) {
      float2 pr[KB];
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const int e = e0 + k * kThreads;
        const int ec = e < n ? e : n - 1;
        const int h = ec / hw, v2 = ec - h * hw;
        pr[k] = *(const float2*)(src + (size_t)h * W + 2 * v2);
      }
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const int e = e0 + k * kThreads;
        if (e < n) {
          const int h = e / hw, v2 = e - h * hw;
          P[(h + 1) * PW + 2 * v2 + 1] = pr[k].x;
          P[(h + 1) * PW + 2 * v2 + 2] = pr[k].y;
        }
      }
    }
  } else {
    for (int e = threadIdx.x; e < H * W; e += kThreads) {
      const int h = e / W, v = e - h * W;
      P[(h + 1) * PW + v + 1] = src[(size_t)h * W + v];
    }
  }
}

__device__ __forceinline__ void put_map(uint16_t* p, float v) { *p = f2bf(v); }
__device__ __forceinline__ void put_map(float* p, float v) { *p = v; }

// Column strips over halo-padded LDS planes (pitch W + 2): a task is (plane slot, column v,
// strip of kStrip rows); walking down the strip with a sliding 3x3 register window
// win[a][b] = P[(h + a) * PW + v + b] = input (h + a - 1, v + b - 1) reads 3 LDS values per row.
constexpr int kStrip = 7;

template <class F>
__device__ __forceinline__ void walk_strip(const float* P, int PW, int v, int h0, int h1, F&& f) {
  float win[3][3];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 3; ++b) win[a][b] = P[(h0 + a) * PW + v + b];
  for (int h = h0; h < h1; ++h) {
#pragma unroll
    for (int b = 0; b < 3; ++b) win[2][b] = P[(h + 2) * PW + v + b];
    f(h, win);
#pragma unroll
    for (int b = 0; b < 3; ++b) {
      win[0][b] = win[1][b];
      win[1][b] = win[2][b];
    }
  }
}

// Planes staged together so that a plane's strips (W * ceil(H / kStrip) tasks) fill the block.
__host__ __device__ inline int mix_tasks_per_plane(int H, int W) {
  return W * ((H + kStrip - 1) / kStrip);
}
__host__ __device__ inline int mix_planes_together(int H, int W) {
  const int t = mix_tasks_per_plane(H, W);
  const int sp = t >= kThreads ? 1 : kThreads / t;
  return sp > 4 ? 4 : sp;
}

// Mix adjoint and dWmix partials of whole planes: workgroup (c, q) takes planes (b, c) for
// b = q*PB .. q*PB + PB - 1, SP at a time; each is staged in LDS with a one-pixel zero halo (dy and
// z), then every pixel's 9 neighbours (from the strip's register window) give both
// g[h,v] = sum_{u,t} W[u][t] dy[h-u+1, v-t+1] (written as bf16) and the dWmix terms
// z[h,v] dy[h-u+1, v-t+1] (fp64 per thread over all its planes). The 9 sums are then reduced over
// the wave by shuffles and over the 4 waves in a fixed order into the workgroup's partial
// partW[c][q][9] (z may be null: no partials). Maps are bf16 or fp32 (TM); g has their type.
template <typename TM>
__global__ void __launch_bounds__(kThreads) k_mix_bwd_planes(
    const TM* __restrict__ dy, const TM* __restrict__ z, const float* __restrict__ w9,
    TM* __restrict__ g, double* __restrict__ partW, int B, int C, int H, int W, int PB) {
  extern __shared__ __attribute__((aligned(16))) float smem_f[];
  __shared__ double wsum[4][9];
  const int c = blockIdx.x, q = blockIdx.y;
  const int PW = W + 2, plane = (H + 2) * PW;
  const int SP = mix_planes_together(H, W), tpp = mix_tasks_per_plane(H, W);
  const int nstrip = (H + kStrip - 1) / kStrip;
  float w[9];
#pragma unroll
  for (int k = 0; k < 9; ++k) w[k] = w9[c * 9 + k];
  double acc[9];
#pragma unroll
  for (int k = 0; k < 9; ++k) acc[k] = 0.0;
  const int b0 = q * PB, b1 = min(B, (q + 1) * PB);
  for (int bs = b0; bs < b1; bs += SP) {
    if (bs > b0) __syncthreads();  // every thread is done with the previous planes
    const int np = min(SP, b1 - bs);
    for (int j = 0; j < np; ++j) {
      const size_t base = ((size_t)(bs + j) * C + c) * H * W;
      stage_plane<TM>(dy + base, smem_f + (2 * j) * plane, H, W);
      if (z) stage_plane<TM>(z + base, smem_f + (2 * j + 1) * plane, H, W);
    }
    __syncthreads();
    for (int task = threadIdx.x; task < np * tpp; task += kThreads) {
      const int j = task / tpp, r = task - j * tpp;
      const int sidx = r / W, v = r - sidx * W;
      const float* Dp = smem_f + (2 * j) * plane;
      const float* Zp = smem_f + (2 * j + 1) * plane;
      TM* gp = g + ((size_t)(bs + j) * C + c) * H * W;
      const int h0 = sidx * kStrip, h1 = min(H, h0 + kStrip);
      walk_strip(Dp, PW, v, h0, h1, [&](int h, const float (&win)[3][3]) {
        // dy[h-u+1][v-t+1] = win[2-u][2-t]
        float gv = 0.f;
#pragma unroll
        for (int k = 0; k < 9; ++k) gv = fmaf(w[k], win[2 - k / 3][2 - k % 3], gv);
        put_map(gp + (size_t)h * W + v, gv);
        if (z) {
          const double zv = Zp[(h + 1) * PW + v + 1];
#pragma unroll
          for (int k = 0; k < 9; ++k) acc[k] += zv * (double)win[2 - k / 3][2 - k % 3];
        }
      });
    }
  }
  if (!z) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < 9; ++k) {
    double v = acc[k];
    for (int off = 32; off > 0; off >>= 1) v += __shfl_down(v, off, 64);
    if (lane == 0) wsum[wave][k] = v;
  }
  __syncthreads();
  if (threadIdx.x < 9) {
    const int k = threadIdx.x;
    partW[((size_t)c * gridDim.y + q) * 9 + k] = ((wsum[0][k] + wsum[1][k]) + wsum[2][k]) + wsum[3][k];
  }
}

// y = mix3x3(z) of whole planes (fp32 sums; bf16 maps rounded to nearest even): workgroup q takes
// planes q*SP .. + SP - 1 (the stand-alone mix pass after a forward that wrote z).
template <typename TM>
__global__ void __launch_bounds__(kThreads) k_mix_fwd_planes(
    const TM* __restrict__ z, const float* __restrict__ w9, TM* __restrict__ y, int C,
    int H, int W, int planes) {
  extern __shared__ __attribute__((aligned(16))) float smem_f[];
  const int PW = W + 2, plane = (H + 2) * PW;
  const int SP = mix_planes_together(H, W), tpp = mix_tasks_per_plane(H, W);
  const int p0 = blockIdx.x * SP, np = min(SP, planes - p0);
  for (int j = 0; j < np; ++j)
    stage_plane<TM>(z + (size_t)(p0 + j) * H * W, smem_f + j * plane, H, W);
  __syncthreads();
  for (int task = threadIdx.x; task < np * tpp; task += kThreads) {
    const int j = task / tpp, r = task - j * tpp;
    const int sidx = r / W, v = r - sidx * W;
    const int c = (p0 + j) % C;
    float w[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) w[k] = w9[c * 9 + k];
    TM* yp = y + (size_t)(p0 + j) * H * W;
    const int h0 = sidx * kStrip, h1 = min(H, h0 + kStrip);
    walk_strip(smem_f + j * plane, PW, v, h0, h1, [&](int h, const float (&win)[3][3]) {
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < 9; ++k) acc = fmaf(w[k], win[k / 3][k % 3], acc);
      put_map(yp + (size_t)h * W + v, acc);
    });
  }
}

// Direct 3x3 mix passes for NCHW planes of even width (any height): no staging and no barrier
// before the arithmetic. A lane takes a column pair (2cp, 2cp + 1) and a run of kMixRun rows
// h0 .. h0 + kMixRun - 1 of one plane and loads its own pixel pair of the kMixRun + 2 rows
// h0 - 1 .. h0 + kMixRun (a 4-byte word for bf16, a float2 for fp32) through a buffer resource
// spanning the plane: the rows above and below the plane fall outside it and read as zero, which
// is the mix's zero padding, and stores outside it are dropped, so no access needs a branch. The
// lanes of a wave hold consecutive column pairs of whole row runs, so the neighbouring pixels
// 2cp - 1 and 2cp + 2 come from the lanes beside it by DPP wave shifts (lanes at a row's ends take
// zero); rows wider than 64 pairs are split over waves and the two lanes at a wave's ends load the
// pixel beyond it themselves. n[r][j] below is pixel (h0 - 1 + r, 2cp - 1 + j), j = 0..3. A wave
// takes kMixNpw small planes (one wave unit each) of one channel with all their loads in flight at
// once; larger planes are split into chunks of four wave units, one workgroup per chunk.
//   forward: y[h][v] = sum_{u,t} W[u][t] z[h+u-1][v+t-1]            [gecl.asia reading notes,
//   adjoint: g[h][v] = sum_{u,t} W[u][t] dy[h-u+1][v-t+1]             "Method" point 3: the
//   weights: dW[u][t] = sum_{h,v} z[h][v] dy[h-u+1][v-t+1]            inter-block 3x3 mix]
// (k = 3u + t in a fixed fmaf order per output, the same order as the plane-staged kernels, so the
// two give equal bits; bf16 outputs round to nearest even). dW: fp32 sums over a lane's pixels of
// one plane (at most 2 kMixRun products of map values per weight), then fp64 over its planes and
// over the wave in a fixed order (through LDS: four lanes per weight add 16 lanes' values each,
// then the four sums are paired); a wave of small planes leaves partial partW[c][q][9] (planes
// b = q kMixNpw ..), a chunk the sum of its four waves in order, partW[c][b][chunk][9];
// k_bwd_reduce adds them per channel in order.
constexpr int kMixRun = 7;
constexpr int kMixNpw = 2;  // small planes of one channel per wave

// Wave units per plane: a wave holds 64 / CP whole row runs (CP = W / 2 <= 64 pairs per row) or
// 64 pairs of one run.
__host__ __device__ inline int mix_direct_wpp(int H, int W) {
  const int CP = W / 2, nseg = (H + kMixRun - 1) / kMixRun;
  if (CP <= 64) {
    const int spw = 64 / CP;
    return (nseg + spw - 1) / spw;
  }
  return nseg * ((CP + 63) / 64);
}
__host__ __device__ inline int mix_direct_chunks(int H, int W) {
  const int wpp = mix_direct_wpp(H, W);
  return wpp == 1 ? 1 : (wpp + 3) / 4;
}

// Planes the direct passes take: even width, byte offsets (rows above included) below 2^31.
inline bool mix_direct_ok(int H, int W) {
  return (W & 1) == 0 && (long long)(H + 2) * W * 4 < (1LL << 30);
}

typedef float mix_v2f __attribute__((ext_vector_type(2)));
typedef __bf16 mix_v2bf __attribute__((ext_vector_type(2)));

// A plane as a raw buffer of `bytes` bytes: loads past it read 0, stores past it are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t plane_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

template <typename TM>
struct MixPair;
template <>
struct MixPair<uint16_t> {  // two bf16 pixels as one word
  typedef uint32_t T;
  static __device__ __forceinline__ T load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
  }
  static __device__ __forceinline__ float lo(T w) { return __uint_as_float(w << 16); }
  static __device__ __forceinline__ float hi(T w) { return __uint_as_float(w & 0xffff0000u); }
  static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t off, float a,
                                               float b) {
    const uint32_t v = __builtin_bit_cast(uint32_t, __builtin_convertvector((mix_v2f{a, b}), mix_v2bf));
    __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, 0);
  }
};
template <>
struct MixPair<float> {
  typedef float2 T;
  static __device__ __forceinline__ T load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
  }
  static __device__ __forceinline__ float lo(T w) { return w.x; }
  static __device__ __forceinline__ float hi(T w) { return w.y; }
  static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t off, float a,
                                               float b) {
    typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2v, make_float2(a, b)), r,
                                          (int)off, 0, 0);
  }
};

// x of lane i - 1 (CTRL 0x138, wave_shr:1) or i + 1 (0x130, wave_shl:1); 0 past the wave's ends
template <int CTRL>
__device__ __forceinline__ float dpp_wave_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
}
// x + (x of the lane given by a quad permutation)
template <int CTRL>
__device__ __forceinline__ double add_quad_f64(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)b, CTRL, 0xf, 0xf, true);
  const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), CTRL, 0xf, 0xf, true);
  return x + __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}

struct MixDirectArgs {
  const void* src;   // z (forward) or dy (adjoint)
  const void* zs;    // adjoint: saved z for the weight partials, or null
  const float* w9;   // (C, 3, 3)
  void* dst;         // y or g
  double* partW;     // adjoint with zs: see above
  int B, C, H, W, wpp, chunks;
};

template <typename TM, bool ADJ>
__global__ void __launch_bounds__(kThreads) k_mix_direct(MixDirectArgs a) {
  typedef MixPair<TM> MP;
  typedef typename MP::T PT;
  constexpr int R = kMixRun, NPW = kMixNpw, PS = (int)sizeof(PT);
  __shared__ __attribute__((aligned(16))) double red[ADJ ? 4 * 9 * 64 : 1];
  __shared__ double wsum[4][9];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int CP = a.W >> 1, nseg = (a.H + R - 1) / R;
  const bool small = a.wpp == 1;  // uniform
  const int groups = (a.B + NPW - 1) / NPW;
  // this wave (all uniform): planes (b0 + j, c), j < nb, and wave unit wu of each
  int c, b0, nb, wu, chunk = 0, wi = 0;
  bool wlive;
  if (small) {
    wi = blockIdx.x * 4 + wave;
    wlive = wi < a.C * groups;
    c = wlive ? wi / groups : 0;
    b0 = wlive ? (wi - c * groups) * NPW : 0;
    nb = min(NPW, a.B - b0);
    wu = 0;
  } else {
    const int p = blockIdx.x / a.chunks;
    chunk = blockIdx.x - p * a.chunks;
    wu = chunk * 4 + wave;
    wlive = wu < a.wpp;
    b0 = p / a.C;
    c = p - b0 * a.C;
    nb = 1;
  }
  int seg, cp;
  bool task;
  if (CP <= 64) {
    const int spw = 64 / CP, s = lane / CP;
    seg = wu * spw + s;
    cp = lane - s * CP;
    task = wlive && s < spw && seg < nseg;
  } else {
    const int wpr = (CP + 63) / 64;
    seg = wu / wpr;
    cp = (wu - seg * wpr) * 64 + lane;
    task = wlive && cp < CP;
  }
  if (!task) cp = 0;
  const int h0 = seg * R;
  const uint32_t rowb = (uint32_t)a.W * sizeof(TM);
  const int pbytes = a.H * (int)rowb;
  // byte offset of this lane's pair in row h0 - 1 + r: a row above the plane wraps to an offset
  // >= 2^31, past the plane; lanes without a task start at 2^31
  const uint32_t off0 = task ? (uint32_t)(h0 - 1) * rowb + (uint32_t)(cp * PS) : 0x80000000u;
  float w[9];
#pragma unroll
  for (int k = 0; k < 9; ++k) w[k] = a.w9[c * 9 + k];
  const size_t pstride = (size_t)a.C * a.H * a.W;  // elements from image b to b + 1
  const size_t pbase = ((size_t)b0 * a.C + c) * a.H * a.W;
  // every load of the wave's planes in flight before the first sum
  PT own[NPW][R + 2];
  PT zr[NPW][R];
#pragma unroll
  for (int j = 0; j < NPW; ++j) {
    if (j >= nb) break;  // uniform
    const __amdgpu_buffer_rsrc_t rs = plane_rsrc((const TM*)a.src + pbase + j * pstride, pbytes);
#pragma unroll
    for (int r = 0; r < R + 2; ++r) own[j][r] = MP::load(rs, off0 + r * rowb);
    if constexpr (ADJ) {
      if (a.zs) {
        const __amdgpu_buffer_rsrc_t rz = plane_rsrc((const TM*)a.zs + pbase + j * pstride, pbytes);
#pragma unroll
        for (int i = 0; i < R; ++i) zr[j][i] = MP::load(rz, off0 + (i + 1) * rowb);
      }
    }
  }
  double dacc[9];
#pragma unroll
  for (int k = 0; k < 9; ++k) dacc[k] = 0.0;
#pragma unroll
  for (int j = 0; j < NPW; ++j) {
    if (j >= nb) break;  // uniform
    float n[R + 2][4];
#pragma unroll
    for (int r = 0; r < R + 2; ++r) {
      n[r][1] = MP::lo(own[j][r]);
      n[r][2] = MP::hi(own[j][r]);
      // the pixels beside the pair: the neighbouring lanes' pairs
      const float lft = dpp_wave_f32<0x138>(n[r][2]);
      const float rgt = dpp_wave_f32<0x130>(n[r][1]);
      n[r][0] = cp > 0 ? lft : 0.f;
      n[r][3] = cp < CP - 1 ? rgt : 0.f;
    }
    if (CP > 64) {  // uniform: rows split over waves; the end lanes load across the split
      const __amdgpu_buffer_rsrc_t rs = plane_rsrc((const TM*)a.src + pbase + j * pstride, pbytes);
#pragma unroll
      for (int r = 0; r < R + 2; ++r) {
        if (task && lane == 0 && cp > 0) n[r][0] = MP::hi(MP::load(rs, off0 + r * rowb - PS));
        if (task && lane == 63 && cp < CP - 1) n[r][3] = MP::lo(MP::load(rs, off0 + r * rowb + PS));
      }
    }
    const __amdgpu_buffer_rsrc_t rd = plane_rsrc((const TM*)a.dst + pbase + j * pstride, pbytes);
    float fw[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) fw[k] = 0.f;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      float o0 = 0.f, o1 = 0.f;
#pragma unroll
      for (int k = 0; k < 9; ++k) {
        const int u = k / 3, tt = k % 3;
        if constexpr (ADJ) {  // dy[h-u+1][v-t+1]: row i + 2 - u, column (of pixel 2cp) 2 - t
          o0 = fmaf(w[k], n[i + 2 - u][2 - tt], o0);
          o1 = fmaf(w[k], n[i + 2 - u][3 - tt], o1);
        } else {              // z[h+u-1][v+t-1]: row i + u, column t
          o0 = fmaf(w[k], n[i + u][tt], o0);
          o1 = fmaf(w[k], n[i + u][tt + 1], o1);
        }
      }
      MP::store(rd, off0 + (i + 1) * rowb, o0, o1);  // rows past the plane are dropped
      if constexpr (ADJ) {
        if (a.zs) {
          const float z0 = MP::lo(zr[j][i]), z1 = MP::hi(zr[j][i]);
#pragma unroll
          for (int k = 0; k < 9; ++k) {
            const int u = k / 3, tt = k % 3;
            fw[k] = fmaf(z0, n[i + 2 - u][2 - tt], fw[k]);
            fw[k] = fmaf(z1, n[i + 2 - u][3 - tt], fw[k]);
          }
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 9; ++k) dacc[k] += (double)fw[k];
  }
  if constexpr (ADJ) {
    if (!a.zs) return;  // uniform
    // wave sums: red[wave][k][lane]; lane 4k + q adds lanes 16q .. 16q + 15 of weight k in order,
    // then (q0 + q1) + (q2 + q3) by quad permutations, left in lane 4k
    double* rw = red + wave * 9 * 64;
#pragma unroll
    for (int k = 0; k < 9; ++k) rw[k * 64 + lane] = dacc[k];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int kk = min(lane >> 2, 8), q = lane & 3;
    const double* rp = rw + kk * 64 + 16 * q;
    double sum = 0.0;
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const double2 v = *(const double2*)(rp + i);
      sum += v.x;
      sum += v.y;
    }
    sum = add_quad_f64<0xB1>(sum);  // quad_perm [1, 0, 3, 2]
    sum = add_quad_f64<0x4E>(sum);  // quad_perm [2, 3, 0, 1]
    const bool holder = lane < 36 && q == 0;
    if (small) {
      if (holder && wlive) a.partW[(size_t)wi * 9 + kk] = sum;
      return;
    }
    if (holder) wsum[wave][kk] = sum;
    __syncthreads();
    if (threadIdx.x < 9) {
      const int k = threadIdx.x;
      a.partW[(((size_t)c * a.B + b0) * a.chunks + chunk) * 9 + k] =
          ((wsum[0][k] + wsum[1][k]) + wsum[2][k]) + wsum[3][k];
    }
  }
}

template <typename TM, bool ADJ>
hipError_t launch_mix_direct(const TM* src, const TM* zs, const float* w9, TM* dst, double* partW,
                             int B, int C, int H, int W, hipStream_t st) {
  if (!mix_direct_ok(H, W) || B < 1 || C < 1 || H < 1) return hipErrorInvalidValue;
  MixDirectArgs a{};
  a.src = src;
  a.zs = zs;
  a.w9 = w9;
  a.dst = dst;
  a.partW = partW;
  a.B = B;
  a.C = C;
  a.H = H;
  a.W = W;
  a.wpp = mix_direct_wpp(H, W);
  a.chunks = mix_direct_chunks(H, W);
  const long long waves = (long long)C * ((B + kMixNpw - 1) / kMixNpw);
  const long long grid = a.wpp == 1 ? (waves + 3) / 4 : (long long)B * C * a.chunks;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_mix_direct<TM, ADJ>), dim3((unsigned)grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <typename TM>
hipError_t launch_mix_fwd_planes(const TM* z, const float* w9, TM* y, int B, int C, int H, int W,
                                 hipStream_t st) {
  if (mix_direct_ok(H, W)) return launch_mix_direct<TM, false>(z, nullptr, w9, y, nullptr, B, C, H, W, st);
  const int sp = mix_planes_together(H, W);
  const size_t lds = (size_t)sp * (H + 2) * (W + 2) * sizeof(float);
  if (lds > 64 * 1024) return hipErrorInvalidValue;
  const int planes = B * C;
  hipLaunchKernelGGL(k_mix_fwd_planes<TM>, dim3((planes + sp - 1) / sp), dim3(kThreads),
                     (unsigned)lds, st, z, w9, y, C, H, W, planes);
  return hipGetLastError();
}

hipError_t launch_mix_fwd_planes_bf16(const uint16_t* z, const float* w9, uint16_t* y, int B,
                                      int C, int H, int W, hipStream_t st) {
  return launch_mix_fwd_planes<uint16_t>(z, w9, y, B, C, H, W, st);
}

hipError_t launch_mix_fwd_planes_f32(const float* z, const float* w9, float* y, int B, int C,
                                     int H, int W, hipStream_t st) {
  return launch_mix_fwd_planes<float>(z, w9, y, B, C, H, W, st);
}

// fp32 NCHW mix pass after a forward that wrote z: whole planes staged in LDS when they fit (up to
// 150 KB for one plane, so 128 x 128 planes stage too), else the per-pixel kernel.
hipError_t launch_mix_fwd_f32_route(const float* z, const float* w9, float* y, int B, int C,
                                    int H, int W, hipStream_t st) {
  if (mix_direct_ok(H, W))
    return launch_mix_direct<float, false>(z, nullptr, w9, y, nullptr, B, C, H, W, st);
  const int sp = mix_planes_together(H, W);
  const size_t lds = (size_t)sp * (H + 2) * (W + 2) * sizeof(float);
  if (lds > 150 * 1024) return launch_mix_fwd(z, w9, y, 0, B, C, H, W, 0, st);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)k_mix_fwd_planes<float>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int planes = B * C;
  hipLaunchKernelGGL(k_mix_fwd_planes<float>, dim3((planes + sp - 1) / sp), dim3(kThreads),
                     (unsigned)lds, st, z, w9, y, C, H, W, planes);
  return hipGetLastError();
}

size_t mix_planes_lds_bytes(int H, int W) {
  return (size_t)2 * mix_planes_together(H, W) * (H + 2) * (W + 2) * sizeof(float);
}

static int mix_planes_per_group(int B) { return B < 8 ? B : 8; }

bool mix_bwd_pass_ok(int H, int W) {
  return mix_direct_ok(H, W) || mix_planes_lds_bytes(H, W) <= 64 * 1024;
}

int mix_bwd_parts(int B, int H, int W) {
  if (mix_direct_ok(H, W))
    return mix_direct_wpp(H, W) == 1 ? (B + kMixNpw - 1) / kMixNpw : B * mix_direct_chunks(H, W);
  const int pb = mix_planes_per_group(B);
  return (B + pb - 1) / pb;
}

template <typename TM>
hipError_t launch_mix_bwd_planes(const TM* dy, const TM* z, const float* w9, TM* g, double* partW,
                                 int B, int C, int H, int W, hipStream_t st) {
  if (mix_direct_ok(H, W)) return launch_mix_direct<TM, true>(dy, z, w9, g, partW, B, C, H, W, st);
  const size_t lds = mix_planes_lds_bytes(H, W);
  if (lds > 64 * 1024) return hipErrorInvalidValue;
  const int pb = mix_planes_per_group(B);
  hipLaunchKernelGGL(k_mix_bwd_planes<TM>, dim3(C, (B + pb - 1) / pb), dim3(kThreads),
                     (unsigned)lds, st, dy, z, w9, g, partW, B, C, H, W, pb);
  return hipGetLastError();
}

hipError_t launch_mix_bwd_planes_bf16(const uint16_t* dy, const uint16_t* z, const float* w9,
                                      uint16_t* g, double* partW, int B, int C, int H, int W,
                                      hipStream_t st) {
  return launch_mix_bwd_planes<uint16_t>(dy, z, w9, g, partW, B, C, H, W, st);
}

hipError_t launch_mix_bwd_planes_f32(const float* dy, const float* z, const float* w9, float* g,
                                     double* partW, int B, int C, int H, int W, hipStream_t st) {
  return launch_mix_bwd_planes<float>(dy, z, w9, g, partW, B, C, H, W, st);
}

}  // namespace wbmm
