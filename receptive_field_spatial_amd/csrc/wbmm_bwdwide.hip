// Backward for windows wider than 16 (17 <= w <= 32): fp32 or bf16 maps, table or cached matrix,
// NCHW or NHWC, ragged and padded maps, any grid offset. By the chain rule (forward
// z = M_c . X_c per window, y = mix3x3(z)) [gecl.asia reading notes, "Core Idea", "Method"]:
//   G  = mix adjoint of dy (the stand-alone mix passes; G = dy without a mix), dWmix with it;
//   dX = M_c^T . G_c: the forward contraction on G with the table rotated by 180 degrees
//        (M(rot180 T) = M(T)^T), or the general contraction reading the cached matrix
//        transposed;
//   dT_c[dy][dx] = sum over windows and row pairs y1 - y2 = dy of the diagonal x1 - x2 = dx of
//        G_n[y1][:] (x) X_n[y2][:]: the row-pair form of the w <= 16 kernels, here on
//        v_mfma_f32_32x32x2f32 tiles (a whole window row of up to 32 pixels per tile side) with
//        the windows as K.
// dT kernel: workgroup (c, chunk) stages 4 windows of G and X (zero outside the map and past the
// window) in LDS as 32 x 32 pixel blocks; wave q takes the row offsets dy = q, q + 4, ... and for
// each accumulates its tile over the valid row pairs and the 4 windows (2 per instruction), then
// sums the tile's diagonals in fp64 (each diagonal in a fixed order) into the chunk's partial;
// k_bwd_reduce adds the partials in a fixed order.
#include "wbmm_device.hpp"
#include "wbmm_launch.hpp"

namespace wbmm {

namespace {

constexpr int kWideNW = 4;   // windows per workgroup chunk
constexpr int kWideP = 32;   // staged block side

typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ v16f mfma32x2(float a, float b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Element copy T_r[c][q] = T[c][L - 1 - q] (E = float or bf16 bits): the rotated table.
template <typename E>
__global__ void __launch_bounds__(kThreads) k_rot_table(const E* __restrict__ T, E* __restrict__ Tr,
                                                        int C, int L) {
  const size_t total = (size_t)C * L;
  for (size_t e = (size_t)blockIdx.x * kThreads + threadIdx.x; e < total;
       e += (size_t)gridDim.x * kThreads) {
    const size_t c = e / L, q = e - c * L;
    Tr[e] = T[c * L + (L - 1 - q)];
  }
}

struct DtWideArgs {
  int B, C, H, W, w, layout, oy, ox;
  int nWx, nWin;     // windows per grid row, per image
  int nwin_ch;       // windows per channel (B * nWin)
  int chunks;        // ceil(nwin_ch / kWideNW)
  const void* g;     // G map
  const void* x;     // X map
  double* partT;     // [C][chunks][L]
};

template <typename TM>
__global__ void __launch_bounds__(kThreads) k_dt_wide(DtWideArgs a) {
  __shared__ __attribute__((aligned(16))) float Gs[kWideNW][kWideP][kWideP];
  __shared__ __attribute__((aligned(16))) float Xs[kWideNW][kWideP][kWideP];
  __shared__ float scr[4][kWideP][kWideP + 1];
  const int c = blockIdx.y, chunk = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int w = a.w, L1 = 2 * w - 1, L = L1 * L1;
  const TM* g = (const TM*)a.g;
  const TM* x = (const TM*)a.x;
  // stage: element (window kn, row y, column v) of both maps, zero outside the window, the map
  // or the channel's windows
  for (int e = threadIdx.x; e < kWideNW * kWideP * kWideP; e += kThreads) {
    const int kn = e / (kWideP * kWideP), rem = e - kn * (kWideP * kWideP);
    const int y = rem / kWideP, v = rem - y * kWideP;
    const int n = chunk * kWideNW + kn;
    float gv = 0.f, xv = 0.f;
    if (n < a.nwin_ch && y < w && v < w) {
      const int b = n / a.nWin, wi = n - b * a.nWin;
      const int wy = wi / a.nWx, wx = wi - wy * a.nWx;
      const int h = wy * w - a.oy + y, col = wx * w - a.ox + v;
      if (h >= 0 && h < a.H && col >= 0 && col < a.W) {
        const size_t off = map_off(a.layout, b, c, h, col, a.C, a.H, a.W);
        gv = load_f32<TM>(g, off);
        xv = load_f32<TM>(x, off);
      }
    }
    Gs[kn][y][v] = gv;
    Xs[kn][y][v] = xv;
  }
  __syncthreads();
  // lane (l32, kh): A row x1 = l32 of window 2 kp + kh; B column x2 = l32 of window 2 kp + kh
  const int l32 = lane & 31, kh = lane >> 5;
  double* part = a.partT + ((size_t)c * a.chunks + chunk) * L;
  float (*S)[kWideP + 1] = scr[wave];
  for (int dyi = wave; dyi < L1; dyi += 4) {  // uniform per wave
    const int dyv = dyi - (w - 1);
    v16f acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
    const int y1a = dyv > 0 ? dyv : 0, y1b = dyv < 0 ? w + dyv : w;
    for (int y1 = y1a; y1 < y1b; ++y1) {
      const int y2 = y1 - dyv;
#pragma unroll
      for (int kp = 0; kp < kWideNW / 2; ++kp) {
        const float av = Gs[2 * kp + kh][y1][l32];
        const float bv = Xs[2 * kp + kh][y2][l32];
        acc = mfma32x2(av, bv, acc);
      }
    }
    // acc[e] is element (x1 = 8 (e / 4) + 4 kh + e % 4, x2 = l32) of the tile
#pragma unroll
    for (int e = 0; e < 16; ++e) S[8 * (e >> 2) + 4 * kh + (e & 3)][l32] = acc[e];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // diagonal dx = lane - (w - 1): x1 - x2 = dx, summed over x1 in order (fp64)
    if (lane < L1) {
      const int dxv = lane - (w - 1);
      double s = 0.0;
      const int x1a = dxv > 0 ? dxv : 0, x1b = dxv < 0 ? w + dxv : w;
      for (int x1 = x1a; x1 < x1b; ++x1) s += (double)S[x1][x1 - dxv];
      part[dyi * L1 + lane] = s;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

size_t al256(size_t v) { return (v + 255) / 256 * 256; }

struct WideGeo {
  int nWx, nWin, nwin_ch, chunks;
};
WideGeo wide_geo(const BwdRequest& r) {
  WideGeo g{};
  g.nWx = (r.W + r.ox + r.w - 1) / r.w;
  const int nWy = (r.H + r.oy + r.w - 1) / r.w;
  g.nWin = g.nWx * nWy;
  g.nwin_ch = r.B * g.nWin;
  g.chunks = (g.nwin_ch + kWideNW - 1) / kWideNW;
  return g;
}

struct WideWs {
  size_t gmap, partW, tab, partT, total;
};
// [G map (mix)] [dWmix partials (mix, NCHW pass)] [rotated table (table input)] [dT partials]
WideWs wide_ws(const BwdRequest& r, size_t esz) {
  const WideGeo g = wide_geo(r);
  const bool mix = r.mixw != nullptr;
  const bool pass = mix && r.layout == 0 && mix_bwd_pass_ok(r.H, r.W);
  WideWs w{};
  const size_t L = (size_t)(2 * r.w - 1) * (2 * r.w - 1);
  w.gmap = 0;
  w.partW = w.gmap + (mix ? al256((size_t)r.B * r.C * r.H * r.W * esz) : 0);
  w.tab = w.partW + (pass ? al256((size_t)r.C * mix_bwd_parts(r.B, r.H, r.W) * 9 * 8) : 0);
  w.partT = w.tab + (r.M ? 0 : al256((size_t)r.C * L * esz));
  w.total = w.partT + al256((size_t)r.C * g.chunks * L * 8);
  return w;
}

template <typename TM>
hipError_t launch_backward_wide_t(const BwdRequest& r, hipStream_t st) {
  constexpr bool kBf16 = sizeof(TM) == 2;
  const WideGeo g = wide_geo(r);
  const WideWs wl = wide_ws(r, sizeof(TM));
  unsigned char* ws = (unsigned char*)r.ws;
  const TM* dy = (const TM*)r.dy;
  const TM* zs = (const TM*)r.zsaved;
  const TM* gmap = dy;
  hipError_t e = hipSuccess;
  const int L = (2 * r.w - 1) * (2 * r.w - 1);
  const bool mix = r.mixw != nullptr;
  const bool pass = mix && r.layout == 0 && mix_bwd_pass_ok(r.H, r.W);
  const int partsW = pass ? mix_bwd_parts(r.B, r.H, r.W) : 0;
  double* partW = (double*)(ws + wl.partW);
  if (mix) {  // G (and the dWmix partials) on the whole map
    TM* gm = (TM*)(ws + wl.gmap);
    if (pass) {
      if constexpr (kBf16)
        e = launch_mix_bwd_planes_bf16(dy, r.dmixw ? zs : nullptr, r.mixw, gm, partW, r.B, r.C,
                                       r.H, r.W, st);
      else
        e = launch_mix_bwd_planes_f32(dy, r.dmixw ? zs : nullptr, r.mixw, gm, partW, r.B, r.C,
                                      r.H, r.W, st);
      if (e != hipSuccess) return e;
    } else {
      e = launch_mix_bwd_data_t<TM>(dy, r.mixw, gm, r.B, r.C, r.H, r.W, r.layout, st);
      if (e != hipSuccess) return e;
      if (r.dmixw) {
        e = launch_mix_bwd_weight_t<TM>(dy, zs, r.dmixw, r.B, r.C, r.H, r.W, r.layout, st);
        if (e != hipSuccess) return e;
      }
    }
    gmap = gm;
  }
  if (r.dx) {  // dX = M^T G: the forward contraction with M^T
    FwdRequest q{};
    q.B = r.B; q.C = r.C; q.H = r.H; q.W = r.W; q.w = r.w; q.layout = r.layout;
    q.in_bf16 = kBf16 ? 1 : 0;
    q.out_bf16 = kBf16 ? 1 : 0;
    q.x = gmap;
    q.y = r.dx;
    q.oy = r.oy;
    q.ox = r.ox;
    TM* tab = (TM*)(ws + wl.tab);
    if (r.M) {  // the general kernel reads the cached matrix transposed
      if constexpr (kBf16) return hipErrorInvalidValue;
      q.M = r.M;
      q.flip = 1;
    } else {
      const size_t n = (size_t)r.C * L;
      const unsigned blocks = (unsigned)((n + kThreads - 1) / kThreads < 4096 ? (n + kThreads - 1) / kThreads : 4096);
      hipLaunchKernelGGL(k_rot_table<TM>, dim3(blocks), dim3(kThreads), 0, st, (const TM*)r.T, tab,
                         r.C, L);
      q.T = tab;
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_forward(q, st);
    if (e != hipSuccess) return e;
  }
  double* partT = (double*)(ws + wl.partT);
  if (r.dT) {
    DtWideArgs a{};
    a.B = r.B; a.C = r.C; a.H = r.H; a.W = r.W; a.w = r.w; a.layout = r.layout;
    a.oy = r.oy; a.ox = r.ox;
    a.nWx = g.nWx; a.nWin = g.nWin; a.nwin_ch = g.nwin_ch; a.chunks = g.chunks;
    a.g = gmap;
    a.x = r.x;
    a.partT = partT;
    hipLaunchKernelGGL(k_dt_wide<TM>, dim3(g.chunks, r.C), dim3(kThreads), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_bwd_reduce2(partT, g.chunks, pass && r.dmixw ? partW : nullptr, partsW, r.C, L,
                              r.dT, pass ? r.dmixw : nullptr, st);
  }
  if (pass && r.dmixw) e = launch_bwd_reduce2(nullptr, 0, partW, partsW, r.C, 0, nullptr, r.dmixw, st);
  return e;
}

}  // namespace

bool wide_backward_ok(const BwdRequest& r) {
  if (r.w <= 16 || r.w > 32 || r.Tsub || r.B < 1 || r.C < 1) return false;
  const WideGeo g = wide_geo(r);
  return g.chunks < 65536 && r.C < 65536 && (long long)r.C * g.chunks < (1LL << 31);
}

size_t backward_wide_workspace(const BwdRequest& r, size_t map_bytes) {
  return wide_backward_ok(r) ? wide_ws(r, map_bytes).total : 0;
}

hipError_t launch_backward_wide(const BwdRequest& r, bool bf16, hipStream_t st) {
  if (!wide_backward_ok(r)) return hipErrorInvalidValue;
  return bf16 ? launch_backward_wide_t<uint16_t>(r, st) : launch_backward_wide_t<float>(r, st);
}

}  // namespace wbmm
