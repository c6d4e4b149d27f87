// bf16 backward for w = 14 on NCHW 28x28 or 56x56 images (maps and table in bf16, fp32 and fp64
// accumulation). By the chain rule (forward z = M_c . X_c per window, y = mix3x3(z)):
//   G  = mix adjoint of dy (a bf16 map; G = dy without a mix), dWmix from dy and z;
//   dX = M_c^T . G_c: the bf16 forward contraction with the table rotated by 180 degrees
//        (M(rot180 T) = M(T)^T), written as bf16;
//   dT_c[k] = sum_{idx[i][j] = k} (G_c . X_c^T)[i][j]: the row-pair form
//        acc_dy[x1][x2] = sum_{windows n} sum_{y1 - y2 = dy} G_n[y1][x1] * X_n[y2][x2]
//        on the bf16 matrix cores with the windows as the K dimension (32 per instruction),
//        whose diagonals x1 - x2 = dx are dT[dy][dx].
// The row-pair kernel stages a unit's 64 windows of G and X transposed in LDS (pixel-major,
// window-minor), so an MFMA operand (8 consecutive windows of one pixel) is one 16-byte read;
// eight waves share a unit's tiles (27 row offsets over 8 waves); each unit leaves one fp64
// partial, summed in a fixed order by k_bwd_reduce.
#include "wbmm_device.hpp"
#include "wbmm_launch.hpp"

namespace wbmm {

namespace {

template <int IW_>
struct DtShape {
  static constexpr int WS = 14, IH = IW_, IW = IW_, D = WS * WS, L1 = 2 * WS - 1, L = L1 * L1;
  static constexpr int NWX = IW / WS, NWIN = NWX * NWX;
  static constexpr int IPW = 16 / NWIN;     // images per wave-unit of 16 windows
  static constexpr int IPU = 4 * IPW;       // images per unit of 64 windows
  static constexpr int PLANE = IH * IW;
  static constexpr int NP = 72;             // bf16 per pixel row of a transposed tile (64 + 8)
  static constexpr int ITEMS = 32 * WS * (WS / 2);  // (window pair, row, pixel pair) of a unit
  static_assert(IW == 28 || IW == 56, "shape");
  static_assert(NP * 2 % 16 == 0, "16-byte operand reads");
};

template <class S>
constexpr int dt_lds_bytes() { return 2 * S::D * S::NP * 2; }

constexpr int kDtWaves = 8;                 // waves per unit
constexpr int kDtThreads = 64 * kDtWaves;
constexpr int kDtSlots = 4;                 // row offsets per wave (27 over 8 waves)

// Row-offset slots of wave Q: offsets ordered 0, +1, -1, +2, -2, ... dealt in a snake so the
// eight waves get near-equal MFMA counts (WS - |dy| row pairs per offset).
template <int WS, int Q, int J>
struct DtSlot {
  static constexpr int T = kDtWaves * J + ((J & 1) ? kDtWaves - 1 - Q : Q);
  static constexpr bool valid = T < 2 * WS - 1;
  static constexpr int dy = T == 0 ? 0 : ((T & 1) ? (T + 1) / 2 : -(T / 2));
};

struct DtArgs {
  int B, C, groups;
  const uint16_t* g;  // G (bf16 map)
  const uint16_t* x;  // X (bf16 map)
  double* partT;      // [C * groups][L]
};

// One wave's row-pair contraction over the unit's 64 windows and its diagonal sums.
template <class S, int Q>
__device__ __forceinline__ void dt_wave(const uint16_t* Gt, const uint16_t* Xt, double* scr,
                                        double* pT, int lane) {
  constexpr int WS = S::WS, DD = WS * WS;
  const int m = lane & 15, grp = lane >> 4;
  const int mc = m < WS ? m : WS - 1;  // MFMA rows/columns 14, 15 are never read
  v4f acc[kDtSlots];
#pragma unroll
  for (int j = 0; j < kDtSlots; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
  // A[x1][n] = G_n[y1][x1] (row x1 = m), B[n][x2] = X_n[y2][x2] (column x2 = m): lane group grp
  // feeds windows k0 + 8 grp .. + 7 of K step k0
  const uint16_t* ga = Gt + mc * S::NP + 8 * grp;
  const uint16_t* xb = Xt + mc * S::NP + 8 * grp;
#define WBMM_DTB_SLOT(J)                                                            \
  if constexpr (DtSlot<WS, Q, J>::valid) {                                          \
    constexpr int dy = DtSlot<WS, Q, J>::dy;                                        \
    _Pragma("unroll") for (int y1 = (dy > 0 ? dy : 0); y1 < (dy < 0 ? WS + dy : WS); ++y1) { \
      const int y2 = y1 - dy;                                                       \
      _Pragma("unroll") for (int k0 = 0; k0 < 64; k0 += 32) {                       \
        const u32x4 av = *(const u32x4*)(ga + y1 * WS * S::NP + k0);                \
        const u32x4 bv = *(const u32x4*)(xb + y2 * WS * S::NP + k0);                \
        acc[J] = mfma_bf16(av, bv, acc[J]);                                         \
      }                                                                             \
    }                                                                               \
  }
  WBMM_DTB_SLOT(0) WBMM_DTB_SLOT(1) WBMM_DTB_SLOT(2) WBMM_DTB_SLOT(3)
#undef WBMM_DTB_SLOT
  __syncthreads();  // every wave is done with the tiles: the scratch reuses them
  // acc[J][r] is element (x1 = 4 grp + r, x2 = m) of slot J's tile; elements outside the WS x WS
  // tile go to a per-lane dump slot, so no store is conditional
  const int dump = kDtSlots * DD + lane;
  static_assert(!DtSlot<WS, Q, kDtSlots>::valid, "every row offset has a slot");
#define WBMM_DTB_PUT(J)                                                            \
  if constexpr (DtSlot<WS, Q, J>::valid) {                                         \
    _Pragma("unroll") for (int r = 0; r < 4; ++r) {                                \
      const int x1 = 4 * grp + r;                                                  \
      scr[(x1 < WS && m < WS) ? J * DD + x1 * WS + m : dump] = (double)acc[J][r];  \
    }                                                                              \
  }
  WBMM_DTB_PUT(0) WBMM_DTB_PUT(1) WBMM_DTB_PUT(2) WBMM_DTB_PUT(3)
#undef WBMM_DTB_PUT
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // diagonal dx = dd - (WS-1) of each tile: lane halves h sum x1 in [7h, 7h + 7), then add in a
  // fixed order
  constexpr int HALF = (WS + 1) / 2;
  const int h = lane >> 5, dd = lane & 31, dxv = dd - (WS - 1);
#define WBMM_DTB_SUM(J)                                                        \
  if constexpr (DtSlot<WS, Q, J>::valid) {                                     \
    double s = 0.0;                                                            \
    _Pragma("unroll") for (int k = 0; k < HALF; ++k) {                         \
      const int x1 = h * HALF + k, xb2 = x1 - dxv;                             \
      const bool ok = dd < S::L1 && x1 < WS && xb2 >= 0 && xb2 < WS;           \
      const double v = scr[ok ? J * DD + x1 * WS + xb2 : J * DD];              \
      s += ok ? v : 0.0;                                                       \
    }                                                                          \
    const double o = __shfl_down(s, 32, 64);                                   \
    if (lane < S::L1) pT[(DtSlot<WS, Q, J>::dy + WS - 1) * S::L1 + lane] = s + o; \
  }
  WBMM_DTB_SUM(0) WBMM_DTB_SUM(1) WBMM_DTB_SUM(2) WBMM_DTB_SUM(3)
#undef WBMM_DTB_SUM
}

// One workgroup (8 waves) per unit of 64 windows (whole images) of one channel.
template <class S>
__global__ void __launch_bounds__(kDtThreads) k_dt_bf16(DtArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem_h[];
  uint16_t* Gt = smem_h;             // [D][NP]: G of pixel p, window n at p * NP + n
  uint16_t* Xt = smem_h + S::D * S::NP;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int u = blockIdx.x;
  const int c = u / a.groups;
  const int img0 = (u - c * a.groups) * S::IPU;

  // ---- stage: item (window pair wp, row y, pixel pair xp) loads pixels 2xp, 2xp+1 of row y of
  //      windows 2wp and 2wp+1 (4 bytes each) and writes each pixel's two windows as one 4-byte
  //      LDS word; windows past the batch are 0. All loads of a lane are in flight before its
  //      writes.
  constexpr int SB = (S::ITEMS + kDtThreads - 1) / kDtThreads;
  uint32_t gv[SB][2], xv[SB][2];
#pragma unroll
  for (int s = 0; s < SB; ++s) {
    const int e = s * kDtThreads + threadIdx.x;
    const int wp = e / (S::WS * S::WS / 2), rem = e - wp * (S::WS * S::WS / 2);
    const int y = rem / (S::WS / 2), xp = rem - y * (S::WS / 2);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int n = 2 * wp + h;
      const int im = n / S::NWIN, k = n - im * S::NWIN;
      const bool in = e < S::ITEMS && img0 + im < a.B;
      const size_t off = in ? ((size_t)(img0 + im) * a.C + c) * S::PLANE +
                                  ((k / S::NWX) * S::WS + y) * S::IW + (k % S::NWX) * S::WS + 2 * xp
                            : 0;
      const uint32_t g2 = *(const uint32_t*)(a.g + off);
      const uint32_t x2 = *(const uint32_t*)(a.x + off);
      gv[s][h] = in ? g2 : 0u;
      xv[s][h] = in ? x2 : 0u;
    }
  }
#pragma unroll
  for (int s = 0; s < SB; ++s) {
    const int e = s * kDtThreads + threadIdx.x;
    if (e >= S::ITEMS) break;
    const int wp = e / (S::WS * S::WS / 2), rem = e - wp * (S::WS * S::WS / 2);
    const int y = rem / (S::WS / 2), xp = rem - y * (S::WS / 2);
    const int p = y * S::WS + 2 * xp;
    // pixel p: (window 2wp, window 2wp+1) = the low halves; pixel p+1: the high halves
    uint32_t* g32 = (uint32_t*)(Gt + p * S::NP + 2 * wp);
    uint32_t* x32 = (uint32_t*)(Xt + p * S::NP + 2 * wp);
    g32[0] = (gv[s][0] & 0xffffu) | (gv[s][1] << 16);
    g32[S::NP / 2] = (gv[s][0] >> 16) | (gv[s][1] & 0xffff0000u);
    x32[0] = (xv[s][0] & 0xffffu) | (xv[s][1] << 16);
    x32[S::NP / 2] = (xv[s][0] >> 16) | (xv[s][1] & 0xffff0000u);
  }
  __syncthreads();

  double* scr = (double*)smem_h + wave * (kDtSlots * S::D + 64);
  double* pT = a.partT + (size_t)u * S::L;
  switch (wave) {
    case 0: dt_wave<S, 0>(Gt, Xt, scr, pT, lane); break;
    case 1: dt_wave<S, 1>(Gt, Xt, scr, pT, lane); break;
    case 2: dt_wave<S, 2>(Gt, Xt, scr, pT, lane); break;
    case 3: dt_wave<S, 3>(Gt, Xt, scr, pT, lane); break;
    case 4: dt_wave<S, 4>(Gt, Xt, scr, pT, lane); break;
    case 5: dt_wave<S, 5>(Gt, Xt, scr, pT, lane); break;
    case 6: dt_wave<S, 6>(Gt, Xt, scr, pT, lane); break;
    default: dt_wave<S, 7>(Gt, Xt, scr, pT, lane); break;
  }
}

using D28 = DtShape<28>;
using D56 = DtShape<56>;
// the diagonal-sum scratch (8 waves x (4 tiles + a dump row) of doubles) fits in the tiles
static_assert(kDtWaves * (kDtSlots * 196 + 64) * 8 <= dt_lds_bytes<D28>(), "scratch");

template <class S>
int dt_groups(int B) { return (B + S::IPU - 1) / S::IPU; }

template <class S>
hipError_t launch_dt(const uint16_t* g, const uint16_t* x, double* partT, int B, int C,
                     hipStream_t st) {
  DtArgs a{};
  a.B = B;
  a.C = C;
  a.groups = dt_groups<S>(B);
  a.g = g;
  a.x = x;
  a.partT = partT;
  const int lds = dt_lds_bytes<S>();
  hipError_t e = hipFuncSetAttribute((const void*)k_dt_bf16<S>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  return launch_main(k_dt_bf16<S>, dim3(C * a.groups), dim3(kDtThreads), lds, st, a);
}

size_t al256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

bool bf16_backward_ok(int B, int C, int H, int W, int w, int layout) {
  return layout == 0 && w == 14 && H == W && (H == 28 || H == 56) && B >= 1 && C >= 1 &&
         (long long)C * ((B + 3) / 4 + 1) < (1LL << 31);
}

namespace {
// The request for the general kernels (bf16 data behind the map and table pointers).
BwdRequest general_request(const BwdBf16Request& q) {
  BwdRequest r{};
  r.B = q.B; r.C = q.C; r.H = q.H; r.W = q.W; r.w = q.w; r.layout = q.layout;
  r.x = (const float*)q.x; r.T = (const float*)q.T; r.mixw = q.mixw;
  r.zsaved = (const float*)q.zsaved; r.dy = (const float*)q.dy; r.dx = (float*)q.dx;
  r.dT = q.dT; r.dmixw = q.dmixw; r.ws = q.ws;
  return r;
}
}  // namespace

bool bf16_backward_plan_ok(int B, int C, int H, int W, int w, int layout) {
  if (bf16_backward_ok(B, C, H, W, w, layout)) return true;
  static const float dummy = 0.f;
  BwdRequest r{};
  r.B = B; r.C = C; r.H = H; r.W = W; r.w = w; r.layout = layout;
  r.x = r.T = r.dy = &dummy;
  return backward_plan_ok(r);
}

// Fast shapes: [G map (bf16), dWmix partials (fp64, per plane): with a mix] [dT partials (fp64)];
// other shapes: the general kernels' layout.
size_t bf16_backward_workspace(int B, int C, int H, int W, int w, int layout, int has_mix) {
  if (!bf16_backward_ok(B, C, H, W, w, layout)) {
    static const float dummy = 0.f;
    BwdRequest r{};
    r.B = B; r.C = C; r.H = H; r.W = W; r.w = w; r.layout = layout;
    r.x = r.T = r.dy = &dummy;
    r.mixw = has_mix ? &dummy : nullptr;
    r.zsaved = has_mix ? &dummy : nullptr;
    return backward_bf16_general_workspace(r);
  }
  const int groups = H == 28 ? dt_groups<D28>(B) : dt_groups<D56>(B);
  const size_t mixpart =
      has_mix ? al256((size_t)B * C * H * W * 2) + al256((size_t)C * mix_bwd_parts(B, H, W) * 9 * 8)
              : 0;
  return mixpart + al256((size_t)C * groups * 729 * 8);
}

hipError_t launch_backward_bf16(const BwdBf16Request& r, hipStream_t st) {
  if (!bf16_backward_ok(r.B, r.C, r.H, r.W, r.w, r.layout))
    return launch_backward_bf16_general(general_request(r), st);
  unsigned char* ws = (unsigned char*)r.ws;
  const bool mix = r.mixw != nullptr;
  const uint16_t* g = r.dy;
  hipError_t e = hipSuccess;
  const size_t gmap = mix ? al256((size_t)r.B * r.C * r.H * r.W * 2) : 0;
  const int partsW = mix ? mix_bwd_parts(r.B, r.H, r.W) : 0;
  const size_t mixpart = mix ? gmap + al256((size_t)r.C * partsW * 9 * 8) : 0;
  double* partW = mix ? (double*)(ws + gmap) : nullptr;
  float* dmixw = mix ? r.dmixw : nullptr;
  if (mix) {  // G and the dWmix partials in one pass over dy and z
    uint16_t* gm = (uint16_t*)ws;
    e = launch_mix_bwd_planes_bf16(r.dy, dmixw ? r.zsaved : nullptr, r.mixw, gm, partW, r.B, r.C,
                                   r.H, r.W, st);
    if (e != hipSuccess) return e;
    g = gm;
  }
  if (r.dx) {
    e = launch_bf16_transposed_contraction(g, r.T, r.dx, r.B, r.C, r.H, st);
    if (e != hipSuccess) return e;
  }
  if (r.dT) {
    double* partT = (double*)(ws + mixpart);
    const int groups = r.H == 28 ? dt_groups<D28>(r.B) : dt_groups<D56>(r.B);
    e = r.H == 28 ? launch_dt<D28>(g, r.x, partT, r.B, r.C, st)
                  : launch_dt<D56>(g, r.x, partT, r.B, r.C, st);
    if (e != hipSuccess) return e;
    // dT and dWmix partials summed in one launch
    return launch_bwd_reduce2(partT, groups, partW, partsW, r.C, 729, r.dT, dmixw, st);
  }
  if (dmixw) e = launch_bwd_reduce2(nullptr, 0, partW, partsW, r.C, 0, nullptr, dmixw, st);
  return e;
}

}  // namespace wbmm
