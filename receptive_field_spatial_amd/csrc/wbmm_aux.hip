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
__global__ void __launch_bounds__(kThreads) k_mix_fwd(const float* __restrict__ z,
                                                      const float* __restrict__ w9, void* y,
                                                      int out_bf16, int B, int C, int H, int W,
                                                      int layout) {
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
  if (dT) {
    for (int q = threadIdx.x; q < L; q += kThreads) {
      const double* p = partT + (size_t)c * parts * L + q;
      double s = 0.0;
      for (int k = 0; k < parts; ++k) s += p[(size_t)k * L];
      dT[(size_t)c * L + q] = (float)s;
    }
  }
  if (dmixw && threadIdx.x < 9) {
    const double* p = partW + (size_t)c * parts * 9 + threadIdx.x;
    double s = 0.0;
    for (int k = 0; k < parts; ++k) s += p[(size_t)k * 9];
    dmixw[c * 9 + threadIdx.x] = (float)s;
  }
}

hipError_t launch_bwd_reduce(const double* partT, const double* partW, int parts, int C, int L,
                             float* dT, float* dmixw, hipStream_t st) {
  hipLaunchKernelGGL(k_bwd_reduce, dim3(C), dim3(kThreads), 0, st, partT, partW, parts, L, dT,
                     dmixw);
  return hipGetLastError();
}

hipError_t launch_mix_fwd(const float* z, const float* w9, void* y, int out_bf16, int B, int C,
                          int H, int W, int layout, hipStream_t st) {
  const size_t n = (size_t)B * C * H * W;
  hipLaunchKernelGGL(k_mix_fwd, dim3(grid_for(n)), dim3(kThreads), 0, st, z, w9, y, out_bf16, B,
                     C, H, W, layout);
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

hipError_t launch_mix_bwd_data_bf16(const uint16_t* dy, const float* w9, uint16_t* dz, int B,
                                    int C, int H, int W, hipStream_t st) {
  const size_t n = (size_t)B * C * H * W;
  hipLaunchKernelGGL(k_mix_bwd_data<uint16_t>, dim3(grid_for(n)), dim3(kThreads), 0, st, dy, w9,
                     dz, B, C, H, W, 0);
  return hipGetLastError();
}

hipError_t launch_mix_bwd_weight_bf16(const uint16_t* dy, const uint16_t* z, float* dw9, int B,
                                      int C, int H, int W, hipStream_t st) {
  hipLaunchKernelGGL(k_mix_bwd_weight<uint16_t>, dim3(C), dim3(kThreads), 0, st, dy, z, dw9, B, C,
                     H, W, 0);
  return hipGetLastError();
}

}  // namespace wbmm
