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
template <typename E>
__global__ void __launch_bounds__(kThreads) k_fold(const E* __restrict__ Min,
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

// dT[c][q] = sum over workgroups k (in order) of partT[c][k][q]; the same for the 9 dWmix values.
__global__ void __launch_bounds__(kThreads) k_bwd_reduce(const double* __restrict__ partT,
                                                         const double* __restrict__ partW,
                                                         int parts, int L, float* __restrict__ dT,
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
  if (dT) {
    for (int q = threadIdx.x; q < L; q += kThreads)
      dT[(size_t)c * L + q] = (float)sum(partT + (size_t)c * parts * L + q, (size_t)L, parts);
  }
  if (dmixw && threadIdx.x < 9)
    dmixw[c * 9 + threadIdx.x] = (float)sum(partW + (size_t)c * parts * 9 + threadIdx.x, 9, parts);
}

hipError_t launch_bwd_reduce(const double* partT, const double* partW, int parts, int C, int L,
                             float* dT, float* dmixw, hipStream_t st) {
  hipLaunchKernelGGL(k_bwd_reduce, dim3(C), dim3(kThreads), 0, st, partT, partW, parts, L, dT,
                     dmixw);
  return hipGetLastError();
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

template <typename TM>
hipError_t launch_mix_fwd_planes(const TM* z, const float* w9, TM* y, int B, int C, int H, int W,
                                 hipStream_t st) {
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

int mix_planes_per_group(int B) { return B < 8 ? B : 8; }

template <typename TM>
hipError_t launch_mix_bwd_planes(const TM* dy, const TM* z, const float* w9, TM* g, double* partW,
                                 int B, int C, int H, int W, hipStream_t st) {
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
